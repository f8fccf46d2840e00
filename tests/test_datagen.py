"""The seeded input generator: shapes, determinism, outlier recipe, the greedy pair plan."""
import numpy as np
import pytest

import datagen


def test_round_to_bf16_exact_and_idempotent():
    x = np.array([1.0, 1.0 + 2 ** -9, 1.0 + 3 * 2 ** -9, -2.5e3, 1e-3])
    r = datagen.round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -7
    assert np.array_equal(datagen.round_to_bf16(r), r)
    # below 2^-126 the bf16 grid is 2^-133 (subnormals)
    sub = datagen.round_to_bf16(np.array([1e-39, 3e-40, -2.0 ** -140]))
    assert np.allclose(sub / 2.0 ** -133, np.rint(sub / 2.0 ** -133), atol=0)
    assert sub[0] == 11 * 2.0 ** -133 and sub[2] == 0.0
    datagen.bf16_bits(sub)
    bits = datagen.bf16_bits(r)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back.astype(np.float64), r)


def test_tiny_workload():
    wl = datagen.make("tiny")
    assert wl.x.shape == (16, 128) and wl.w.shape == (128, 128)
    assert np.abs(wl.x[:, 5]).mean() > 10 * np.abs(np.delete(wl.x, 5, axis=1)).mean()
    wl2 = datagen.make("tiny")
    assert np.array_equal(wl.x, wl2.x) and np.array_equal(wl.w, wl2.w)


def test_q_proj_outlier_recipe_small():
    wl = datagen.make("q_proj", M=256, K=1024, N=64)
    x = wl.x
    col = np.abs(x).mean(axis=0)
    assert (col > 20).sum() == 8
    n_spikes = int(round(1e-4 * 256 * 1024))
    # spikes are x1000 on N(0,1) entries: outside the outlier channels no normal
    # entry exceeds 10, and all but ~1% of spikes do
    normal_cols = col <= 20
    big = (np.abs(x[:, normal_cols]) > 10).sum()
    assert 0.9 * n_spikes <= big <= n_spikes
    assert np.array_equal(datagen.round_to_bf16(x), x)


def test_greedy_plan_invariants():
    for seed in range(6):
        rng = np.random.default_rng([seed, 0])
        plan = datagen.greedy_pair_plan(rng, 128, 8, 64)
        assert len(plan) == 8
        assert len(plan[0]) == 64
        seen = set()
        for layer in plan:
            ch = [c for p in layer for c in p]
            assert len(ch) == len(set(ch))          # disjoint inside the layer
            assert 60 <= len(layer) <= 64
            for p in layer:
                assert p[0] < p[1]
                assert p not in seen                # never reused across layers
                seen.add(p)


def test_givens_plan_arrays_deterministic():
    p1, t1, b1 = datagen.givens_plan(3, 256)
    p2, t2, b2 = datagen.givens_plan(3, 256)
    assert p1.shape == (2, 8, 64, 2) and t1.shape == (2, 8, 64) and b1.shape == (256,)
    assert np.array_equal(p1, p2) and np.array_equal(t1, t2) and np.array_equal(b1, b2)
    assert np.all(np.abs(t1) <= np.pi + 1e-6)
    p3, _, _ = datagen.givens_plan(4, 256)
    assert not np.array_equal(p1, p3)


def test_unknown_workload():
    with pytest.raises(KeyError):
        datagen.make("nope")
