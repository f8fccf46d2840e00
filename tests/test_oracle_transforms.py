"""Oracle pins for the rotations: closed forms, invariants, hand-worked examples."""
import json
import math
import os

import numpy as np
import pytest

import oracle


def _kron_hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 128, 512])
def test_hadamard_orthogonal(n):
    H = oracle.hadamard(n)
    assert np.array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", [2, 8, 128, 1024, 4096])
def test_hadamard_equals_sylvester_recursion(n):
    assert np.array_equal(oracle.hadamard(n), _kron_hadamard(n))


def test_hadamard_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hadamard_sylvester.json")))
    for key, n in (("H2", 2), ("H4", 4), ("H8", 8)):
        assert np.array_equal(oracle.hadamard(n), np.array(g[key], dtype=float))


def test_hadamard_rows_and_column_sums():
    n = 256
    H = oracle.hadamard(n)
    # ones . H = n e_0 (only the first Walsh function has nonzero mean)
    assert np.array_equal(np.ones(n) @ H, n * np.eye(n)[0])
    # normalized block squares to the identity (symmetric and orthogonal)
    Hn = oracle.hadamard_block(n)
    assert np.allclose(Hn @ Hn, np.eye(n), atol=1e-13)


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard(12)


def _givens_spec(rng, K, layers=3):
    G = K // 128
    pairs = np.full((G, layers, 64, 2), 0xFF, dtype=np.uint8)
    theta = rng.uniform(-math.pi, math.pi, size=(G, layers, 64)).astype(np.float32)
    for gi in range(G):
        for l in range(layers):
            perm = rng.permutation(128)
            npairs = 64 - l  # leave some empty slots
            for s in range(npairs):
                i, j = sorted((int(perm[2 * s]), int(perm[2 * s + 1])))
                pairs[gi, l, s] = (i, j)
    beta = rng.normal(0, 0.1, size=K).astype(np.float32)
    return {"kind": "givens", "pairs": pairs, "theta": theta, "beta": beta}


def test_givens_layer_orthogonal_and_norm_preserving():
    rng = np.random.default_rng(1)
    spec = _givens_spec(rng, 128)
    Gm = oracle.givens_layer(128, spec["pairs"][0, 0], spec["theta"][0, 0].astype(np.float64))
    assert np.allclose(Gm.T @ Gm, np.eye(128), atol=1e-14)
    x = rng.standard_normal(128)
    assert abs(np.linalg.norm(x @ Gm) - np.linalg.norm(x)) < 1e-12


def test_givens_pairs_in_a_layer_commute():
    rng = np.random.default_rng(2)
    spec = _givens_spec(rng, 128)
    pairs = spec["pairs"][0, 0]
    th = spec["theta"][0, 0].astype(np.float64)
    order = rng.permutation(64)
    A = oracle.givens_layer(128, pairs, th)
    B = oracle.givens_layer(128, pairs[order], th[order])
    assert np.array_equal(A, B)
    # and equal to the product of single-pair rotations in any order
    P = np.eye(128)
    for s in order:
        P = P @ oracle.givens_layer(128, pairs[s:s + 1], th[s:s + 1])
    assert np.allclose(P, A, atol=1e-14)


def test_givens_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "givens_example.json")))
    pairs = np.array(g["pairs"], dtype=np.uint8)
    for case in g["cases"]:
        R = oracle.givens_group_rotation(pairs, np.array(case["theta"]), g=g["g"])
        y = np.array(case["x"], dtype=float) @ R
        assert np.allclose(y, case["expected"], atol=1e-12), (y, case["expected"])


def test_givens_alpha_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "givens_example.json")))["alpha_case"]
    # a 128-channel group with the 4-channel example embedded in channels 0..3
    pairs = np.full((1, 2, 64, 2), 0xFF, dtype=np.uint8)
    pairs[0, 0, 0] = (0, 1)
    pairs[0, 1, 0] = (1, 2)
    theta = np.zeros((1, 2, 64), dtype=np.float32)
    beta = np.zeros(128, dtype=np.float32)
    beta[:4] = g["beta"]
    spec = {"kind": "givens", "pairs": pairs, "theta": theta, "beta": beta}
    x = np.zeros((1, 128))
    x[0, :4] = g["x"]
    xt = oracle.transform_act(x, spec)
    assert np.allclose(xt[0, :4], g["expected_act"], rtol=1e-7)
    # weight side multiplies by alpha instead
    w = np.zeros((128, 1))
    w[:4, 0] = g["x"]
    wt = oracle.transform_weight(w, spec)
    assert np.allclose(wt[:4, 0], [4, 3, 5, 3.5], rtol=1e-7)


@pytest.mark.parametrize("kind", ["h128", "h512", "givens"])
def test_transform_pair_preserves_product(kind):
    """(X T)(T_w W) = X W: the equivalence the whole method rests on."""
    rng = np.random.default_rng(3)
    K, M, N = 512, 9, 7
    if kind == "givens":
        spec = _givens_spec(rng, K)
    else:
        spec = {"kind": "hadamard", "block": int(kind[1:])}
    X = rng.standard_normal((M, K))
    W = rng.standard_normal((K, N))
    Y0 = X @ W
    Y1 = oracle.transform_act(X, spec) @ oracle.transform_weight(W, spec)
    assert np.linalg.norm(Y1 - Y0) / np.linalg.norm(Y0) < 1e-12


@pytest.mark.parametrize("kind", ["h128", "h4096", "givens"])
def test_transform_then_inverse_roundtrip(kind):
    rng = np.random.default_rng(4)
    K = 4096 if kind == "h4096" else 256
    spec = _givens_spec(rng, K) if kind == "givens" else {"kind": "hadamard", "block": int(kind[1:])}
    X = rng.standard_normal((5, K))
    Xt = oracle.transform_act(X, spec)
    # inverse of the activation transform is the transpose of the weight transform
    back = np.empty_like(Xt)
    for k0, k1, Tw in oracle.weight_transform_blocks(spec, K):
        back[:, k0:k1] = Xt[:, k0:k1] @ Tw
    assert np.max(np.abs(back - X)) < 1e-6
    assert np.max(np.abs(back - X)) < 1e-12


def test_block_transform_is_blockwise():
    """A block-128 transform mixes channels only inside their 128-block."""
    rng = np.random.default_rng(5)
    X = np.zeros((1, 512))
    X[0, 130] = 1.0
    Xt = oracle.transform_act(X, {"kind": "hadamard", "block": 128})
    nz = np.nonzero(np.abs(Xt[0]) > 0)[0]
    assert nz.min() == 128 and nz.max() == 255
    # e_i maps to row i of H / sqrt(b)
    assert np.allclose(Xt[0, 128:256], oracle.hadamard(128)[2] / math.sqrt(128))
    del rng


def test_rotation_spreads_a_spike():
    """A single spike becomes flat: max|x_tilde| = |spike| / sqrt(b) (QuIP# page 2.1 energy spreading)."""
    X = np.zeros((1, 128))
    X[0, 17] = 1000.0
    Xt = oracle.transform_act(X, {"kind": "hadamard", "block": 128})
    assert np.allclose(np.abs(Xt), 1000.0 / math.sqrt(128))
