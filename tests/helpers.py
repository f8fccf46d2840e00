"""Test helpers shared by the oracle tests and the GPU parity tests.

Nothing here computes the method: only conversions between a workload
description and the oracle's transform spec, and comparison bookkeeping.
"""
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
    assert n <= max(1, max_frac * g.size) or n / g.size <= max_frac, f"{n} of {g.size} codes differ"
    return n, g.size
