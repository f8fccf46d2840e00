"""Oracle pins for the INT4 quantizers and the packing."""
import json
import os

import numpy as np
import pytest

import oracle


def _golden(golden_dir, name):
    return json.load(open(os.path.join(golden_dir, name)))


def test_group_quant_golden(golden_dir):
    g = _golden(golden_dir, "group_quant_example.json")
    x = np.zeros((1, 256))
    for k, v in g["group0_entries"].items():
        x[0, int(k)] = v
    codes, scales, _ = oracle.quantize_groups(x)
    assert np.array_equal(scales[0], g["expected_scales"])
    assert codes[0, :10].tolist() == g["expected_codes_group0_first10"]
    assert not codes[0, 10:].any()
    packed = oracle.pack_int4(codes)
    assert packed[0, :8].tolist() == g["expected_first_bytes"]
    # the whole all-zero second group packs to zero bytes
    assert not packed[0, 64:].any()
    # the same row scaled by a power of two: identical codes, scaled scale
    codes2, scales2, _ = oracle.quantize_groups(x * 0.125)
    assert np.array_equal(codes2, codes)
    assert np.array_equal(scales2, scales * 0.125)


def test_quant_properties_random():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, size=(64, 1))
    x[3, 200] = 5e4  # spike
    codes, scales, ratio = oracle.quantize_groups(x)
    # the symmetric scale keeps codes in [-7, 7]
    assert codes.min() >= -7 and codes.max() <= 7
    xg = x.reshape(64, 4, 128)
    cg = codes.reshape(64, 4, 128).astype(float)
    # the group maximum maps to +-7
    am = np.abs(xg).argmax(axis=2)
    top = np.take_along_axis(cg, am[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(top) == 7)
    # reconstruction error at most half a step
    err = np.abs(xg - scales[:, :, None] * cg)
    assert np.all(err <= scales[:, :, None] / 2 * (1 + 1e-12))
    # odd symmetry
    codes_neg, scales_neg, _ = oracle.quantize_groups(-x)
    assert np.array_equal(codes_neg, -codes)
    assert np.array_equal(scales_neg, scales)


def test_codes_in_range_and_argmax_hits_7():
    """The INT4 container is [-8, 7] (Rotated Runtime Smooth page, problem
    definition), but with the symmetric scale max / 7 the quantizer's image
    is [-7, 7]: -8 never arises, even for groups built to reach it (minimum
    exactly -max, every ratio an exact half, values just above -max), and
    the group's extreme maps to +-7 exactly.  The same holds for the RRS
    per-token quantizer."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((40, 256))
    x[0, :128] = -3.0            # constant negative group: all -7
    x[1, :128] = 0.0
    x[1, 5], x[1, 9] = 2.0, -2.0  # min = -max
    x[2, :128] = np.linspace(-7.0, 7.0, 128)
    x[3, :128] = -np.arange(128) / 127 * 7.0 - 1e-12
    x[4, :128] = (np.arange(128) % 15 - 7) + 0.5  # halves everywhere, max 7.5
    x[5, :] = -np.abs(x[5, :]) * 1e30
    for codes in (oracle.quantize_groups(x)[0], oracle.quantize_rrs(x)[0]):
        assert codes.min() >= -7 and codes.max() <= 7
    codes, scales, _ = oracle.quantize_groups(x)
    assert np.all(codes[0, :128] == -7)
    assert codes[1, 9] == -7 and codes[1, 5] == 7
    xg = np.abs(x.reshape(40, 2, 128))
    cg = np.abs(codes.reshape(40, 2, 128))
    top = np.take_along_axis(cg, xg.argmax(axis=2)[:, :, None], axis=2)
    assert np.all(top == 7)


def test_pack_rejects_minus_8():
    """The packed layout stores the quantizer's domain [-7, 7] only."""
    for bad in (-8, 8):
        c = np.zeros((1, 8), dtype=np.int8)
        c[0, 3] = bad
        with pytest.raises(ValueError):
            oracle.pack_int4(c)
    c = np.concatenate([np.arange(-7, 8), np.arange(7, -8, -1), [0, 0]]).astype(np.int8).reshape(1, 32)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(c)), c)


def test_quant_zero_and_constant_groups():
    x = np.zeros((2, 256))
    x[1, 128:] = -3.0
    codes, scales, _ = oracle.quantize_groups(x)
    assert np.array_equal(scales, [[0, 0], [0, 3.0 / 7]])
    assert not codes[0].any()
    assert np.all(codes[1, 128:] == -7)


def test_quant_rounds_half_to_even():
    # scale 1 exactly (max 7): ratios are exact halves
    x = np.zeros((1, 128))
    x[0, :6] = [0.5, 1.5, 2.5, -0.5, -1.5, 7.0]
    codes, _, _ = oracle.quantize_groups(x)
    assert codes[0, :6].tolist() == [0, 2, 2, 0, -2, 7]


def test_pack_unpack_roundtrip_and_positions():
    rng = np.random.default_rng(8)
    c = rng.integers(-7, 8, size=(5, 256)).astype(np.int8)
    p = oracle.pack_int4(c)
    assert p.shape == (5, 128) and p.dtype == np.uint8
    assert np.array_equal(oracle.unpack_int4(p), c)
    # single codes of a 32-code chunk (words 0-3; pairs (0, 3) and (1, 2)),
    # bytes worked out from the dense FP6 string X = sum_k f_k << 6 k of the
    # pair (0, 3): X[0:32] lies in word 0, X[64:96] in word 3, and of
    # X[32:64] the field offsets 3, 4 go to word 0, offsets 0, 5 to word 3
    row = np.zeros((1, 32), dtype=np.int8)
    row[0, 0] = -1                     # f_0 = 100001b: X bits 0 and 5 -> word 0
    assert oracle.pack_int4(row)[0].tolist() == [0x21, 0, 0, 0] + [0] * 12
    row[0] = 0
    row[0, 1] = -7                     # f_1 = 100111b: X bits 6, 7, 8, 11 -> word 0
    assert oracle.pack_int4(row)[0].tolist() == [0xC0, 0x09, 0, 0] + [0] * 12
    row[0] = 0
    row[0, 7] = -3                     # f_7: X bits 42, 43 (|c|) and 47 (sign) = X[32:64] bits 10, 11, 15
    assert oracle.pack_int4(row)[0].tolist() == [0, 0x84, 0, 0] + [0] * 8 + [0, 0x08, 0, 0]
    row[0] = 0
    row[0, 5] = 7                      # f_5: X bits 30, 31 -> word 0; X bit 32 (offset 2) -> word 3 bit 0
    assert oracle.pack_int4(row)[0].tolist() == [0, 0, 0, 0xC0] + [0] * 8 + [0x01, 0, 0, 0]
    row[0] = 0
    row[0, 26] = -5                    # word 3's code 2 = f_10: X bits 60, 62, 65 -> word 0 bit 28, word 3 bits 30, 1
    assert oracle.pack_int4(row)[0].tolist() == [0, 0, 0, 0x10] + [0] * 8 + [0x02, 0, 0, 0x40]
    row[0] = 0
    row[0, 15] = -2                    # pair (1, 2) never reaches words 0 and 3
    assert oracle.pack_int4(row)[0, :4].tolist() == [0] * 4 and oracle.pack_int4(row)[0, 12:].tolist() == [0] * 4
    # a negative zero (sign bit set, magnitude 0) decodes to 0
    assert oracle.unpack_int4(np.array([[0x20] + [0] * 15], dtype=np.uint8)).tolist() == [[0] * 32]
    with pytest.raises(ValueError):
        oracle.pack_int4(np.array([[8] + [0] * 31]))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.array([[-8] + [0] * 31]))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.zeros((1, 16), dtype=np.int8))  # half a chunk


def _fp6_dense(codes, signed):
    """The 96-bit string sum_k f_k << 6 k of 16 codes' FP6 E2M3 encodings
    (sign bit 5, exponent bits 3-4, mantissa bits 0-2): c / 8 is a
    subnormal (exponent 0, mantissa |c|) for |c| <= 7; u / 8 for u = 8..15
    has exponent 1 and mantissa u - 8, i.e. the 6-bit pattern u."""
    x = 0
    for k, c in enumerate(codes):
        c = int(c)
        f = ((32 if c < 0 else 0) | abs(c)) if signed else c
        x |= f << (6 * k)
    return x


def _open_pair(a, b, signed):
    """The three words of the dense FP6 string from a stored word pair, by the
    mask identity the GEMM applies (two masks, no rotation)."""
    A, C = (0xE79E79E7, 0x9E79E79E) if signed else (0xCF3CF3CF, 0x3CF3CF3C)
    full = 0xFFFFFFFF
    d0, d2 = a & A, b & C
    d1 = (a & ~A & full) | (b & ~C & full)
    return d0 | (d1 << 32) | (d2 << 64)


@pytest.mark.parametrize("signed", [True, False])
def test_packed_pairs_open_into_dense_fp6(signed):
    """Brute force over random rows: every word pair (4 j, 4 j + 3) and
    (4 j + 1, 4 j + 2), opened with the mask identity, is exactly the dense
    FP6 E2M3 string of its 16 codes (the first word's 8, then its
    partner's), and the table uses each bit of both words once."""
    layout = oracle.SIGNED_PAIR_LAYOUT if signed else oracle.UNSIGNED_PAIR_LAYOUT
    assert sorted(pos for code in layout for pos in code) == [(r, b) for r in (0, 1) for b in range(32)]
    rng = np.random.default_rng(10 if signed else 11)
    c = rng.integers(-7, 8, size=(32, 128)) if signed else rng.integers(0, 16, size=(32, 128))
    p = (oracle.pack_int4(c) if signed else oracle.pack_uint4(c)).astype(np.uint64)
    w = p[:, 0::4] | (p[:, 1::4] << np.uint64(8)) | (p[:, 2::4] << np.uint64(16)) | (p[:, 3::4] << np.uint64(24))
    for row in range(32):
        for j in range(4):
            for a, b in ((0, 3), (1, 2)):
                got = _open_pair(int(w[row, 4 * j + a]), int(w[row, 4 * j + b]), signed)
                codes = np.concatenate([c[row, 32 * j + 8 * a:32 * j + 8 * a + 8], c[row, 32 * j + 8 * b:32 * j + 8 * b + 8]])
                assert got == _fp6_dense(codes, signed), (row, j, a)


def test_rrs_golden(golden_dir):
    g = _golden(golden_dir, "rrs_example.json")
    xt = np.zeros((2, 256))
    for r, key in ((0, "row0"), (1, "row1")):
        for k, v in g[key].items():
            xt[r, int(k)] = v
    codes, sa, s, _ = oracle.quantize_rrs(xt)
    assert np.array_equal(s, g["expected_s"])
    assert np.allclose(sa, g["expected_sa"], rtol=1e-15)
    for r, key in ((0, "row0"), (1, "row1")):
        exp = np.zeros(256, dtype=int)
        for k, v in g["expected_codes"][key].items():
            exp[int(k)] = v
        assert codes[r].tolist() == exp.tolist()
    # per-group quantization of the same values differs (row 1, group 1)
    cg, _, _ = oracle.quantize_groups(xt)
    assert cg[1, 128] == 2 and cg[1, 130] == 7


def test_rrs_smoothed_values_in_unit_range():
    """After smoothing every channel lies in [-1, 1] and each group reaches 1 (RRS page: scaled to [-1,1])."""
    rng = np.random.default_rng(9)
    xt = rng.standard_normal((33, 512))
    xt[:, 7] *= 100
    xt[4, 300] = 1e4
    codes, sa, s, ratio = oracle.quantize_rrs(xt)
    z = xt / np.repeat(s, 128)[None, :]
    assert np.abs(z).max() <= 1.0
    assert np.allclose(np.abs(z).reshape(33, 4, 128).max(axis=(0, 2)), 1.0)
    # every token's largest smoothed value maps to +-7
    am = np.abs(z).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(33), am]) == 7)
    assert codes.min() >= -7 and codes.max() <= 7


def test_rrs_identity_quantizer_gives_exact_product():
    """With the rounding replaced by the identity the s_g cancel and Y = X W exactly (RRS main equation)."""
    rng = np.random.default_rng(10)
    M, K, N = 6, 512, 5
    spec = {"kind": "hadamard", "block": 512}
    X = rng.standard_normal((M, K))
    X[:, 3] *= 50
    W = rng.standard_normal((K, N))
    xt = oracle.transform_act(X, spec)
    codes, sa, s, _ = oracle.quantize_rrs(xt, quantizer=lambda r: r)
    wt = oracle.transform_weight(W, spec)
    Y = np.zeros((M, N))
    for gi in range(K // 128):
        sl = slice(gi * 128, (gi + 1) * 128)
        Y += sa[:, gi][:, None] * (codes[:, sl] @ wt[sl, :])
    assert np.linalg.norm(Y - X @ W) / np.linalg.norm(X @ W) < 1e-12


def test_rrs_channel_permutation_invariance():
    """Reordering channel groups of X_tilde and W_tilde together leaves Y unchanged (RRS Figure 4 (1))."""
    rng = np.random.default_rng(11)
    M, K, N = 8, 512, 6
    xt = rng.standard_normal((M, K))
    xt[:, 100] *= 30
    wt = rng.standard_normal((K, N)) * 0.02
    perm_g = rng.permutation(K // 128)
    perm = np.concatenate([np.arange(g * 128, (g + 1) * 128) for g in perm_g])

    def forward(a, w):
        codes, sa, _, _ = oracle.quantize_rrs(a)
        qw, sw, _ = oracle.quantize_groups(w.T)
        return oracle.dequant_gemm(codes, sa, qw, sw)

    assert np.allclose(forward(xt, wt), forward(xt[:, perm], wt[perm, :]), rtol=1e-13, atol=1e-13)


def test_quantize_act_end_to_end_shapes():
    rng = np.random.default_rng(12)
    X = rng.standard_normal((3, 256))
    out = oracle.quantize_act(X, {"kind": "hadamard", "block": 128})
    assert out["qa"].shape == (3, 128) and out["sa"].shape == (3, 2)
    assert np.array_equal(oracle.unpack_int4(out["qa"]), out["codes"])
