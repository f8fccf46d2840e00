"""Edge patterns and a seeded random-shape loop through the C ABI against the
oracle (the same bars as tests/test_parity_gpu.py).

* Two outlier tokens: the Rotated Runtime Smooth page (current limitations,
  item 4) names inputs where only two tokens carry the outliers as rare but
  troublesome for RRS: then those two tokens alone set every group's
  smoothing scale and every other token is smoothed by maxima far above its
  own.  The kernels must still match the oracle there.
* Random shapes: 48 seeded cases over the transforms and modes each shape
  supports (block-128 Hadamard, with and without random signs, larger
  blocks, Rotated Runtime Smooth, Givens): M in [1, 300], K = 128 * [1, 40],
  N in [1, 300] on the small-M kernel, and every eighth case with M in
  [600, 1100], N in [1600, 2300] on the tiled kernel.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402

if torch.cuda.is_available():
    from tests import test_parity_gpu as tp  # noqa: E402


@pytest.mark.parametrize("K,block", [(4096, 4096), (1024, 1024), (2048, 128)])
def test_rrs_two_outlier_tokens(K, block):
    M, N = 512, 64
    rng = np.random.default_rng(K + block)
    x = datagen.outlier_activations(rng, M, K)
    x[7] *= 1.0e4
    x[300] *= -1.0e4
    x = datagen.round_to_bf16(x)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    wl = datagen.Workload(f"two_tokens_{K}_{block}", M, K, N, x, "bf16", w, ("hadamard", block), "rrs", "f32")
    t, xd, qa, sa, aref = tp._quant_parity(wl)
    # the two tokens set every group maximum
    xt = aref["xt"]
    top = np.abs(xt).reshape(M, K // 128, 128).max(axis=2).argmax(axis=0)
    assert set(top.tolist()) <= {7, 300}
    qw, sw, wref = tp._weight_parity(wl, t)
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


def _random_cases():
    rng = np.random.default_rng(20260103)
    cases = []
    for i in range(48):
        big = i % 8 == 7
        M = int(rng.integers(600, 1101)) if big else int(rng.integers(1, 301))
        N = int(rng.integers(1600, 2301)) if big else int(rng.integers(1, 301))
        kind = ["h128", "rrs", "givens", "hblock", "signed"][i % 5]
        if kind == "rrs" or kind == "hblock":
            K = int(rng.choice([512, 1024, 2048, 4096]))
        else:
            K = 128 * int(rng.integers(1, 9 if big else 41))
        xdt = "bf16" if rng.random() < 0.7 else "f32"
        cases.append((f"rand{i}_{kind}_M{M}_K{K}_N{N}_{xdt}", M, K, N, kind, xdt, int(rng.integers(1 << 30))))
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_shapes(case):
    name, M, K, N, kind, xdt, seed = case
    rng = np.random.default_rng(seed)
    x = datagen.outlier_activations(rng, M, K)
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    kw = {}
    if kind == "h128":
        tr, mode = ("hadamard", 128), "group128"
    elif kind == "signed":
        # blocks above 128 need K in {512, ..., 8192}
        block = int(rng.choice([128, 256])) if K in (512, 1024, 2048, 4096, 8192) else 128
        tr, mode = ("hadamard", block), "group128"
        kw = {"signs": datagen.random_signs(seed % 1000, K)}
    elif kind == "rrs":
        tr, mode = ("hadamard", int(rng.choice([128, K]))), "rrs"
    elif kind == "hblock":
        tr, mode = ("hadamard", int(rng.choice([256, 512, K]))), "group128"
    else:
        layers = int(rng.integers(1, 13))
        tr, mode = ("givens", layers), "group128"
        kw = dict(zip(("pairs", "theta", "beta"), datagen.givens_plan(seed % 1000, K, layers=layers)))
    wl = datagen.Workload(name, M, K, N, x, xdt, w, tr, mode, "f32", **kw)
    t, xd, qa, sa, aref = tp._quant_parity(wl)
    qw, sw, wref = tp._weight_parity(wl, t)
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)
