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
