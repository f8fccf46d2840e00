"""Oracle pins for the grouped integer GEMM and the dequantization epilogue."""
import numpy as np

import datagen
import oracle
from tests.helpers import rel_fro, spec_of


def _brute_acc(qa, qw, g=128):
    M, K = qa.shape
    N = qw.shape[0]
    acc = [[[0] * (K // g) for _ in range(N)] for _ in range(M)]
    for m in range(M):
        for n in range(N):
            for k in range(K):
                acc[m][n][k // g] += int(qa[m, k]) * int(qw[n, k])
    return np.array(acc, dtype=np.int64)


def test_group_accumulators_match_python_ints():
    rng = np.random.default_rng(20)
    qa = rng.integers(-7, 8, size=(3, 256)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(4, 256)).astype(np.int8)
    assert np.array_equal(oracle.group_accumulators(qa, qw), _brute_acc(qa, qw))


def test_group_accumulator_bound():
    qa = np.full((1, 128), -7, dtype=np.int8)
    qw = np.full((1, 128), -7, dtype=np.int8)
    acc = oracle.group_accumulators(qa, qw)
    assert acc[0, 0, 0] == 128 * 49 == 6272
    qw[0] = 7
    assert oracle.group_accumulators(qa, qw)[0, 0, 0] == -6272


def test_dequant_gemm_matches_brute_force():
    rng = np.random.default_rng(21)
    qa = rng.integers(-7, 8, size=(3, 384)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(5, 384)).astype(np.int8)
    sa = rng.uniform(0.1, 2, size=(3, 3))
    sw = rng.uniform(0.1, 2, size=(5, 3))
    acc = _brute_acc(qa, qw)
    Y = np.zeros((3, 5))
    for m in range(3):
        for n in range(5):
            Y[m, n] = sum(sa[m, g] * sw[n, g] * acc[m, n, g] for g in range(3))
    assert np.allclose(oracle.dequant_gemm(qa, sa, qw, sw), Y, rtol=1e-14, atol=0)
    # packed path
    Yp = oracle.w4a4_gemm(oracle.pack_int4(qa), sa, oracle.pack_int4(qw), sw, "f64")
    assert np.allclose(Yp, Y, rtol=1e-14, atol=0)


def test_dequant_gemm_scale_isolation():
    """sa = 1 and sw one-hot on a group reproduces that group's integer accumulator."""
    rng = np.random.default_rng(22)
    qa = rng.integers(-8, 8, size=(4, 512)).astype(np.int8)
    qw = rng.integers(-8, 8, size=(6, 512)).astype(np.int8)
    acc = oracle.group_accumulators(qa, qw)
    for g in range(4):
        sw = np.zeros((6, 4))
        sw[:, g] = 1.0
        Y = oracle.dequant_gemm(qa, np.ones((4, 4)), qw, sw)
        assert np.array_equal(Y, acc[:, :, g].astype(float))


def test_output_rounding():
    y = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -3.14159])
    b = oracle.round_bf16(y)
    assert b[0] == 1.0          # tie -> even mantissa
    assert b[1] == 1.0 + 2 ** -7
    assert abs(b[2] - -3.140625) < 1e-12
    f = oracle.round_output(np.array([1 / 3]), "f32")
    assert f[0] == float(np.float32(1 / 3))


def test_rotation_lowers_w4a4_error():
    """Block-Hadamard W4A4 is closer to X W than untransformed W4A4 on outlier activations.

    Block size 1 is the identity transform (H_1 = [1]).  Directional check of
    the pages' outlier-spreading claim (QuIP# page 2.1; RRS page).
    """
    wl = datagen.make("q_proj", seed=0, M=64, K=1024, N=256)
    Y_ref = wl.x @ wl.w.astype(np.float64)
    errs = {}
    for b in (1, 128):
        spec = {"kind": "hadamard", "block": b}
        Y, _, _ = oracle.layer_forward(wl.x, wl.w, spec, "group128", "f64")
        errs[b] = rel_fro(Y, Y_ref)
    assert errs[128] < errs[1]


def test_rrs_lowers_error_vs_plain_per_token():
    """Rotated Runtime Smooth beats per-token INT4 with neither rotation nor smoothing.

    Directional check of the RRS page's claim on outlier-laden activations;
    the per-token baseline is written out here (max over the row / 7).
    """
    for seed in range(2):
        wl = datagen.make("rrs", seed=seed, M=64, K=1024, N=128)
        Y_ref = wl.x @ wl.w.astype(np.float64)
        Y_rrs, _, _ = oracle.layer_forward(wl.x, wl.w, spec_of(wl), "rrs", "f64")
        a = np.abs(wl.x).max(axis=1) / 7
        q = np.clip(np.rint(wl.x / a[:, None]), -8, 7)
        w = oracle.pack_weight(wl.w, {"kind": "hadamard", "block": 1})
        Y_plain = oracle.dequant_gemm(q, np.repeat(a[:, None], 8, axis=1), w["codes"], w["sw"])
        assert rel_fro(Y_rrs, Y_ref) < rel_fro(Y_plain, Y_ref)
