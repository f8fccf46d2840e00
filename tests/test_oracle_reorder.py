"""Pins of the oracle's Rotated Runtime Smooth channel reorder (the Rotated
Runtime Smooth page, Figure 4 (1) and (2)) and of the per-output-channel
weight quantizer it pairs with (the page's experimental setup: weights
per-channel symmetric)."""
import json
import os

import numpy as np
import pytest

import datagen
import oracle
from tests.helpers import rel_fro, spec_of


def test_reorder_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rrs_reorder_example.json")))
    xt = np.array(g["xt"])
    order, m = oracle.rrs_channel_order(xt)
    assert order.tolist() == g["expected_order"]
    assert m.tolist() == g["expected_maxima"]
    codes, sa, s, ratio = oracle.quantize_rrs(xt[:, order], g["group"])
    assert s.tolist() == g["expected_group_scales"]
    assert codes.tolist() == g["expected_codes"]
    assert np.allclose(sa, g["expected_sa"], rtol=1e-15, atol=0)


def test_order_is_stable_descending_permutation():
    rng = np.random.default_rng(3)
    xt = rng.standard_normal((20, 256))
    xt[:, 10] = 5.0
    xt[:, 200] = -5.0       # equal maxima: the lower channel index first
    xt[:, 77] = 0.0         # an all-zero channel sorts last
    order, m = oracle.rrs_channel_order(xt)
    assert sorted(order.tolist()) == list(range(256))
    assert np.all(np.diff(m[order]) <= 0)
    assert order[0] == 10 and order[1] == 200
    assert order[-1] == 77
    # equal maxima keep increasing index everywhere
    mm = m[order]
    eq = np.where(mm[:-1] == mm[1:])[0]
    assert np.all(order[eq] < order[eq + 1])


def test_identity_order_is_plain_rrs():
    rng = np.random.default_rng(4)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, 33, 512))
    spec = {"kind": "hadamard", "block": 512}
    a = oracle.quantize_act(x, spec, "rrs")
    b = oracle.quantize_act(x, spec, "rrs_reorder", order=np.arange(512))
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["sa"], b["sa"])


def test_reorder_leaves_the_product_unchanged():
    """Figure 4 (1): with the quantizer replaced by the identity, the reordered
    path (activations and weights permuted alike, group scales of the
    reordered groups applied per block) returns X W."""
    rng = np.random.default_rng(5)
    M, K, N = 17, 512, 24
    x = datagen.outlier_activations(rng, M, K)
    w = rng.normal(0, 0.02, size=(K, N))
    spec = {"kind": "hadamard", "block": 512}
    xt = oracle.transform_act(x, spec)
    order, _ = oracle.rrs_channel_order(xt)
    _, sa, s, ratio = oracle.quantize_rrs(xt[:, order], 128, quantizer=lambda r: r)
    wt = oracle.transform_weight(w, spec)[order, :]
    y = oracle.dequant_gemm(ratio, sa, wt.T, np.ones((N, K // 128)))
    assert np.allclose(y, x @ w, rtol=0, atol=1e-12 * np.abs(x).sum(axis=1).max() * np.abs(w).max())
    # and a wrong weight order breaks it
    y_bad = oracle.dequant_gemm(ratio, sa, oracle.transform_weight(w, spec).T, np.ones((N, K // 128)))
    assert not np.allclose(y_bad, x @ w, atol=1e-3)


def test_sorted_grouping_minimizes_the_group_scales():
    """Grouping channels in decreasing order of their maxima gives the
    smallest possible sum of group maxima over all partitions into groups of
    equal size (the k-th largest group maximum is at least the element of
    rank g (k - 1) + 1): each channel is divided by a scale as close to its
    own maximum as any grouping allows."""
    rng = np.random.default_rng(8)
    x = datagen.outlier_activations(rng, 64, 1024)
    order, m = oracle.rrs_channel_order(x)
    s_sorted = oracle.quantize_rrs(x[:, order])[2]
    for perm in [np.arange(1024)] + [rng.permutation(1024) for _ in range(20)]:
        s_other = oracle.quantize_rrs(x[:, perm])[2]
        assert s_sorted.sum() <= s_other.sum()
    assert np.array_equal(s_sorted, m[order][::128])  # each group's scale is its first (largest) channel


def test_reorder_equalizes_channel_precision():
    """What the reorder is for: with runtime smoothing and channel outliers
    (no rotation), natural groups divide the ordinary channels sharing a group
    with an outlier by the outlier's maximum, and INT4 flattens them; grouped
    by their maxima every channel keeps its precision.  Mean over channels of
    the relative reconstruction error: about 0.97 -> 0.22 on the outlier recipe.
    (After the full 4096-point rotation the channel maxima are already nearly
    equal and the reorder changes little either way on these inputs.)"""
    def chan_err(xh, x):
        n = np.linalg.norm(x, axis=0)
        return float(np.mean(np.linalg.norm(xh - x, axis=0)[n > 0] / n[n > 0]))
    for seed in (0, 1, 2):
        x = datagen.outlier_activations(np.random.default_rng(seed), 128, 1024)
        order, _ = oracle.rrs_channel_order(x)
        c0, sa0, _, _ = oracle.quantize_rrs(x)
        c1, sa1, _, _ = oracle.quantize_rrs(x[:, order])
        e0 = chan_err(oracle.dequantize(c0, sa0), x)
        e1 = chan_err(oracle.dequantize(c1, sa1), x[:, order])
        assert e1 < 0.5 * e0, (seed, e0, e1)


def test_per_channel_weights_and_code_permutation():
    rng = np.random.default_rng(6)
    K, N = 512, 10
    w = rng.normal(0, 0.02, size=(K, N))
    w[:, 3] = 0.0
    spec = {"kind": "hadamard", "block": 512}
    p = oracle.pack_weight(w, spec, per_channel=True)
    wt = oracle.transform_weight(w, spec)
    scale = np.abs(wt).max(axis=0) / 7
    assert np.array_equal(p["sw"], np.repeat(scale[:, None], K // 128, axis=1))
    assert not p["codes"][3].any() and not p["sw"][3].any()
    nz = scale > 0
    top = np.abs(p["codes"])[nz].max(axis=1)
    assert np.all(top == 7)
    assert np.all(np.abs(wt.T[nz] - p["codes"][nz] * scale[nz, None]) <= scale[nz, None] / 2 * (1 + 1e-12))
    order = rng.permutation(K)
    q = oracle.permute_codes(p["codes"], order)
    assert np.array_equal(q[:, 5], p["codes"][:, order[5]])
    # a permutation of the codes is the quantization of the permuted weights (per-channel scales)
    p2 = oracle.pack_weight(w, spec, per_channel=True)
    c2, s2, _ = oracle.quantize_per_channel(wt[order, :].T)
    assert np.array_equal(c2, q) and np.array_equal(s2, p2["sw"][:, 0])
