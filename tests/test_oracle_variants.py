"""Oracle pins for the transform / quantizer variants: the randomized
(signed) Hadamard transform and dequantization."""
import numpy as np
import pytest

import datagen
import oracle


def _spec(b, signs=None):
    s = {"kind": "hadamard", "block": b}
    if signs is not None:
        s["signs"] = signs
    return s


@pytest.mark.parametrize("b", [128, 512])
def test_signed_hadamard_is_orthogonal_and_preserves_xw(b):
    K = 1024
    signs = datagen.random_signs(3, K)
    rng = np.random.default_rng(1)
    X = rng.standard_normal((5, K))
    W = rng.standard_normal((K, 7))
    for k0, k1, T in oracle.act_transform_blocks(_spec(b, signs), K):
        assert np.allclose(T @ T.T, np.eye(k1 - k0), atol=1e-12)
    Xt = oracle.transform_act(X, _spec(b, signs))
    Wt = oracle.transform_weight(W, _spec(b, signs))
    assert np.allclose(Xt @ Wt, X @ W, rtol=1e-10, atol=1e-9)
    # the transform is invertible: X = Xt R^T block by block
    back = np.empty_like(Xt)
    for k0, k1, T in oracle.act_transform_blocks(_spec(b, signs), K):
        back[:, k0:k1] = Xt[:, k0:k1] @ T.T
    assert np.allclose(back, X, atol=1e-12)


def test_signs_flip_exactly_their_channels():
    K, b = 256, 128
    plain = _spec(b)
    ones = np.ones(K, dtype=np.int8)
    E = np.eye(K)
    # all +1 reduces to the plain transform
    assert np.array_equal(oracle.transform_act(E, _spec(b, ones)), oracle.transform_act(E, plain))
    signs = ones.copy()
    signs[[3, 200]] = -1
    got = oracle.transform_act(E, _spec(b, signs))
    ref = oracle.transform_act(E, plain)
    # basis vector k maps to signs[k] * (row k of H_b / sqrt(b)) inside its block
    assert np.array_equal(got[3], -ref[3]) and np.array_equal(got[200], -ref[200])
    others = [k for k in range(K) if k not in (3, 200)]
    assert np.array_equal(got[others], ref[others])
    # weights: W_tilde = (H / sqrt(b)) diag(signs) W per block, i.e. the sign
    # scales row k of W before the block Hadamard
    got_w = oracle.transform_weight(E, _spec(b, signs))
    ref_w = oracle.transform_weight(np.diag(signs.astype(float)), plain)
    assert np.allclose(got_w, ref_w, atol=1e-15)


def test_signed_workload_flag():
    wl = datagen.make("q_proj", M=4, K=256, N=8, signed=True)
    assert wl.signs.shape == (256,) and set(np.unique(wl.signs)) <= {-1, 1}
    with pytest.raises(ValueError):
        datagen.make("decode", M=1, K=256, N=8, signed=True)
    with pytest.raises(ValueError):
        oracle.transform_act(np.zeros((1, 256)), _spec(128, np.zeros(256)))


def test_dequantize_definition_and_rtn_bound():
    codes = np.array([[1, -7, 0, 7] + [0] * 124 + [3] * 128], dtype=np.int8)
    scales = np.array([[0.5, 0.25]])
    x = oracle.dequantize(codes, scales)
    assert x[0, :4].tolist() == [0.5, -3.5, 0.0, 3.5]
    assert np.all(x[0, 128:] == 0.75)
    # quantize then dequantize: error at most half a step, per group
    rng = np.random.default_rng(4)
    X = rng.standard_normal((6, 384)) * rng.uniform(0.1, 10, size=(6, 1))
    c, s, _ = oracle.quantize_groups(X)
    err = np.abs(oracle.dequantize(c, s) - X)
    assert np.all(err <= np.repeat(s, 128, axis=1) / 2 * (1 + 1e-12))


def test_dequant_output_rounding():
    # 7 * (1 + 2^-23) needs 26 significant bits: fp32 rounds it, exactly once
    s = np.float64(np.float32(1.0 + 2.0 ** -23))
    x = oracle.dequantize(np.full((1, 128), 7, dtype=np.int8), np.array([[s]]))
    r32 = oracle.round_dequant_output(x, "f32")
    assert r32[0, 0] == np.float64(np.float32(7 * s))
    assert r32[0, 0] != x[0, 0]
    rb = oracle.round_dequant_output(x, "bf16")
    assert rb[0, 0] == 7.0  # nearest bf16 of 7.0000008
    with pytest.raises(ValueError):
        oracle.round_dequant_output(x, "f16")


# ---------------------------------------------------------------------------
# Group size as a knob of the same quantizer ([Paro] section 2.3 groups
# channels by 128; 64 and 256 are the neighbouring choices).  Pins: the
# group maximum nests (a 256-group's scale is the larger of its two
# 128-groups', and so on), codes keep the per-group quantizer properties,
# and the grouped integer products add up across group sizes exactly.
# ---------------------------------------------------------------------------

def _outlier_rows(seed, R, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K))
    x[:, rng.choice(K, 5, replace=False)] *= 80.0
    return x


@pytest.mark.parametrize("small,big", [(64, 128), (128, 256), (64, 256)])
def test_group_scales_nest(small, big):
    x = _outlier_rows(4, 9, 1024)
    _, s_small, _ = oracle.quantize_groups(x, small)
    _, s_big, _ = oracle.quantize_groups(x, big)
    r = big // small
    assert s_small.shape == (9, 1024 // small) and s_big.shape == (9, 1024 // big)
    assert np.array_equal(s_big, s_small.reshape(9, -1, r).max(axis=2))


@pytest.mark.parametrize("g", [64, 256])
def test_quantizer_properties_at_other_group_sizes(g):
    x = _outlier_rows(5, 6, 1024)
    x[2, :g] = 0.0                                   # one all-zero group
    codes, s, ratio = oracle.quantize_groups(x, g)
    assert codes.min() >= -7 and codes.max() <= 7
    xg = x.reshape(6, -1, g)
    cg = codes.reshape(6, -1, g)
    for r in range(6):
        for j in range(xg.shape[1]):
            if s[r, j] == 0:
                assert not cg[r, j].any() and not xg[r, j].any()
                continue
            i = np.argmax(np.abs(xg[r, j]))
            assert abs(cg[r, j, i]) == 7                               # the maximum maps to +-7
            assert np.all(np.abs(xg[r, j] - s[r, j] * cg[r, j]) <= s[r, j] / 2 * (1 + 1e-12))
    assert s[2, 0] == 0


def test_group_accumulators_add_up_across_group_sizes():
    rng = np.random.default_rng(6)
    qa = rng.integers(-7, 8, size=(5, 512))
    qw = rng.integers(-7, 8, size=(3, 512))
    a64 = oracle.group_accumulators(qa, qw, 64)
    a128 = oracle.group_accumulators(qa, qw, 128)
    a256 = oracle.group_accumulators(qa, qw, 256)
    assert np.array_equal(a128, a64[:, :, 0::2] + a64[:, :, 1::2])
    assert np.array_equal(a256, a128[:, :, 0::2] + a128[:, :, 1::2])
    # brute force in Python integers at g = 256
    for m in range(5):
        for n in range(3):
            for j in range(2):
                ref = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(256 * j, 256 * j + 256))
                assert a256[m, n, j] == ref


def test_gemm_at_g256_equals_g128_with_shared_scales():
    rng = np.random.default_rng(7)
    M, N, K = 4, 6, 1024
    qa = rng.integers(-7, 8, size=(M, K))
    qw = rng.integers(-7, 8, size=(N, K))
    sa = rng.uniform(0.1, 2.0, size=(M, K // 256))
    sw = rng.uniform(0.1, 2.0, size=(N, K // 256))
    y256 = oracle.dequant_gemm(qa, sa, qw, sw, 256)
    y128 = oracle.dequant_gemm(qa, np.repeat(sa, 2, axis=1), qw, np.repeat(sw, 2, axis=1), 128)
    assert np.allclose(y256, y128, rtol=1e-13, atol=0)
    # the packed entry point takes the group size from the scale shapes
    y = oracle.w4a4_gemm(oracle.pack_int4(qa), sa, oracle.pack_int4(qw), sw, "f64")
    assert np.array_equal(y, y256)


def test_quantize_act_group_size_follows_the_transform():
    X = _outlier_rows(8, 7, 512)
    spec = {"kind": "hadamard", "block": 128}
    a128 = oracle.quantize_act(X, spec, "group128", 128)
    a256 = oracle.quantize_act(X, spec, "group128", 256)
    a64 = oracle.quantize_act(X, spec, "group128", 64)
    assert np.array_equal(a128["xt"], a256["xt"])
    assert np.array_equal(a256["sa"], a128["sa"].reshape(7, -1, 2).max(axis=2))
    assert np.array_equal(a128["sa"], a64["sa"].reshape(7, -1, 2).max(axis=2))
    # dequantization at g = 64 is within half a step of the transformed values
    xh = oracle.dequantize(a64["codes"], a64["sa"], 64)
    assert np.all(np.abs(xh - a64["xt"]) <= np.repeat(a64["sa"], 64, axis=1) / 2 * (1 + 1e-12))


def test_round_bf16_grid():
    """bf16 rounding: 8 significant bits for normal values, ties to even, and
    below 2^-126 the subnormal grid of spacing 2^-133 (the same format as
    fp32 with 16 fewer fraction bits)."""
    t = 2.0 ** -133
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.0, -(1.0 + 2 ** -7 + 2 ** -9),
                  2.0 ** -149, t, 1.5 * t, 2.5 * t, 33.2 * t, 2.0 ** -126 * (1 + 2 ** -8), 0.0])
    want = np.array([1.0, 1.0 + 2 ** -6, 3.0, -(1.0 + 2 ** -7),
                     0.0, t, 2 * t, 2 * t, 33 * t, 2.0 ** -126, 0.0])
    assert np.array_equal(oracle.round_bf16(x), want)
    # every float32 value already on the bf16 grid is unchanged
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 16, size=4000, dtype=np.uint32) << 16
    bits = bits[(bits & 0x7F800000) != 0x7F800000]    # finite values only
    u = bits.view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.round_bf16(u), u)


def test_attention_scores_invariant_under_shared_rotation():
    """(q R)(k R)^T = q k^T for the block Hadamard (plain and signed) applied to
    queries and keys alike: the reason an INT4 KV cache may store keys rotated
    (the OstQuant page, section 3.2: the same Hadamard on queries and keys)."""
    rng = np.random.default_rng(31)
    q = rng.standard_normal((6, 256))
    k = rng.standard_normal((9, 256))
    for spec in ({"kind": "hadamard", "block": 128},
                 {"kind": "hadamard", "block": 128, "signs": np.where(rng.random(256) < 0.5, -1.0, 1.0)},
                 {"kind": "hadamard", "block": 256}):
        s = oracle.transform_act(q, spec) @ oracle.transform_act(k, spec).T
        assert np.allclose(s, q @ k.T, rtol=0, atol=1e-12 * np.abs(q).sum() * np.abs(k).max())
    # a rotation that is not shared breaks it
    s_bad = oracle.transform_act(q, {"kind": "hadamard", "block": 128}) @ k.T
    assert not np.allclose(s_bad, q @ k.T, atol=1e-3)
