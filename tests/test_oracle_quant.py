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
    c = np.arange(-7, 9, dtype=np.int8).reshape(1, 16)
    c[0, -1] = 0
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


def test_pack_unpack_roundtrip_and_order():
    rng = np.random.default_rng(8)
    c = rng.integers(-7, 8, size=(5, 256)).astype(np.int8)
    p = oracle.pack_int4(c)
    assert p.shape == (5, 128) and p.dtype == np.uint8
    assert np.array_equal(oracle.unpack_int4(p), c)
    # magnitude in bits 0-2 of nibble e (low nibble = even e); the sign of
    # code e in bit 3 of nibble e+1, the last code's sign in nibble 0
    word = np.zeros((1, 8), dtype=np.int8)
    word[0, 0] = -1
    assert oracle.pack_int4(word)[0].tolist() == [0x81, 0, 0, 0]
    word[0] = [0, -7, 0, 0, 0, 0, 0, 0]
    assert oracle.pack_int4(word)[0].tolist() == [0x70, 0x08, 0, 0]
    word[0] = [0, 0, 0, 0, 0, 0, 0, -3]
    assert oracle.pack_int4(word)[0].tolist() == [0x08, 0, 0, 0x30]
    word[0] = [7, 0, 0, 0, 0, 0, 0, 0]
    assert oracle.pack_int4(word)[0].tolist() == [0x07, 0, 0, 0]
    # words are independent: the sign bit never crosses a 4-byte boundary
    two = np.zeros((1, 16), dtype=np.int8)
    two[0, 7] = -2
    assert oracle.pack_int4(two)[0].tolist() == [0x08, 0, 0, 0x20, 0, 0, 0, 0]
    # a negative zero (sign bit set, magnitude 0) decodes to 0
    assert oracle.unpack_int4(np.array([[0x08, 0, 0, 0]], dtype=np.uint8)).tolist() == [[0] * 8]
    with pytest.raises(ValueError):
        oracle.pack_int4(np.array([[8, 0, 0, 0, 0, 0, 0, 0]]))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.array([[-8, 0, 0, 0, 0, 0, 0, 0]]))


def test_packed_word_splits_into_sign_magnitude_bytes():
    """A word w of the packed form gives the even codes as the bytes of
    w & 0x87878787 and the odd codes as the bytes of rotr(w, 4) & 0x87878787,
    each byte = sign << 7 | magnitude (brute force over random words)."""
    rng = np.random.default_rng(9)
    c = rng.integers(-7, 8, size=(64, 8)).astype(np.int8)
    p = oracle.pack_int4(c).astype(np.uint32)
    w = p[:, 0] | (p[:, 1] << 8) | (p[:, 2] << 16) | (p[:, 3] << 24)
    def decode(u):
        out = []
        for k in range(4):
            b = (int(u) >> (8 * k)) & 0xFF
            out.append(-(b & 7) if b & 0x80 else (b & 7))
        return out
    for row in range(64):
        wi = int(w[row])
        even = decode(wi & 0x87878787)
        rot = ((wi >> 4) | (wi << 28)) & 0xFFFFFFFF
        odd = decode(rot & 0x87878787)
        assert even == c[row, 0::2].tolist()
        assert odd == c[row, 1::2].tolist()


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
