"""Test helpers shared by the oracle tests and the GPU parity tests.

Nothing here computes the method: only conversions between a workload
description and the oracle's transform spec, and comparison bookkeeping.
"""
import zlib

import numpy as np


def spec_of(wl):
    """Oracle transform spec for a datagen.Workload."""
    kind = wl.transform[0]
    if kind == "hadamard":
        spec = {"kind": "hadamard", "block": int(wl.transform[1])}
        if wl.signs is not None:
            spec["signs"] = wl.signs
        return spec
    return {"kind": "givens", "pairs": wl.pairs, "theta": wl.theta, "beta": wl.beta}


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def tie_distance(ratio):
    """Distance of x/scale from the nearest rounding tie (k + 1/2), in code units."""
    r = np.asarray(ratio, dtype=np.float64)
    return np.abs(np.abs(r - np.floor(r)) - 0.5)


def compare_codes(gpu_codes, oracle_codes, oracle_ratio, tie_eps=1e-4, max_frac=1e-4):
    """Codes must be equal except at near-ties, where they may differ by exactly 1.

    Returns (n_mismatch, n_total); raises AssertionError on any other difference.
    """
    g = np.asarray(gpu_codes, dtype=np.int64)
    o = np.asarray(oracle_codes, dtype=np.int64)
    assert g.shape == o.shape, (g.shape, o.shape)
    diff = g != o
    n = int(diff.sum())
    if n:
        d = np.abs(g - o)[diff]
        assert d.max() == 1, f"code differs by {d.max()}"
        td = tie_distance(oracle_ratio)[diff]
        assert td.max() < tie_eps, f"mismatch away from a tie (distance {td.max():.3g})"
    # at most floor(max_frac * size) codes may differ: none at all below 10^4 codes
    assert n <= int(np.floor(max_frac * g.size)), f"{n} of {g.size} codes differ"
    return n, g.size


def case_seed(name: str) -> int:
    """Seed of a named test case, the same in every process (CRC-32 of the name;
    Python's str hash is salted per process)."""
    return zlib.crc32(name.encode())


def epilogue_error_bound(codes_a, sa, codes_w, sw, group, acc_fn):
    """Element-wise bound on the fp32 epilogue's rounding error for identical codes.

    The device sums G = K / group terms p_g * acc_g in fp32 (acc_g exact
    integers, p_g = sa * sw formed to within about 3 fp32 units in the last
    place), one rounding per term, so by the recursive-summation bound
    |y_fp32 - y_exact| <= (G + 4) * 2^-24 * sum_g |p_g * acc_g|.  ``acc_fn``
    gives the exact integer products of one group (the oracle's).  Returns
    that bound as a float64 [M, N] array.
    """
    ca = np.asarray(codes_a)
    cw = np.asarray(codes_w)
    sa = np.abs(np.asarray(sa, dtype=np.float64))
    sw = np.abs(np.asarray(sw, dtype=np.float64))
    G = ca.shape[1] // group
    A = np.zeros((ca.shape[0], cw.shape[0]))
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        acc = acc_fn(ca[:, sl], cw[:, sl], group)[:, :, 0].astype(np.float64)
        A += np.abs(acc) * (sa[:, g][:, None] * sw[:, g][None, :])
    return (G + 4) * 2.0 ** -24 * A


def assert_gemm_close(y_gpu, y_ref, bound, what, rel=1e-5):
    """|y_gpu - y_ref| <= rel * |y_ref| + bound, element by element, and rel-Frobenius <= rel."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    d = np.abs(y_gpu - y_ref)
    lim = rel * np.abs(y_ref) + bound
    bad = d > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {d.size} outputs off; worst excess "
                           f"{float((d - lim).max()):.3g} at {np.unravel_index(int(np.argmax(d - lim)), d.shape)}")
    err = rel_fro(y_gpu, y_ref)
    assert err <= rel, f"{what}: rel-Frobenius {err:.3g}"
    return err, float((d / np.maximum(lim, 1e-300)).max())
