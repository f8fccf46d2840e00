"""Seeded synthetic inputs for the rotated W4A4 hot path.

This module is shared by the CPU oracle and the HIP path.  It produces input
data only: activations, weights and the Givens rotation plan with its angles
and channel log-scales.  It holds none of the method's arithmetic (no
transform, no quantizer, no GEMM); the only numerics here are the random
draws, the rounding of the draws to the storage dtype, and the greedy pair
selection that builds the rotation plan (an input structure, like a sparsity
pattern).

Workloads (all seeded with numpy's PCG64 ``default_rng``):

* ``tiny``      X 16x128 fp32 ~ N(0,1), channel 5 scaled x50; W 128x128 fp32
                ~ N(0, 0.02); Hadamard block 128; fp32 output.
* ``q_proj``    LLaMA-3-8B q_proj prefill: X 2048x4096 ~ N(0,1), 8 distinct
                random channels x100, round(1e-4*M*K) distinct random entries
                x1000, stored as bf16; W 4096x4096 ~ N(0, 0.02); block
                Hadamard 128; bf16 output.
* ``decode``    ParoQuant-style decode: M in {1,4,16} x 4096 with the q_proj
                outlier recipe; W 4096x4096; per 128-channel group a greedy
                plan of 8 layers x 64 disjoint pairs, theta ~ U[-pi, pi],
                beta ~ N(0, 0.1); bf16 output.
* ``down_proj`` LLaMA-3-8B FFN down_proj: X 4096x14336 ~ N(0,1) with
                round(0.001*K) = 14 channels drawn from Student-t(nu=2)
                instead; W 14336x4096; block Hadamard 128; bf16 output.
* ``rrs``       Rotated Runtime Smooth: X 8192x4096 with the q_proj outlier
                recipe; W 4096x11008; full 4096-point Hadamard, runtime
                group-max smoothing, per-token INT4; bf16 output.
* ``kv``        INT4 KV cache: K/V rows of 4096 tokens x 8 heads x 128
                (head dimension = group), the q_proj outlier recipe, a
                block-128 Hadamard per head; quantize and dequantize only
                (no weights).

``random_signs(seed, K)`` draws the +-1 diagonal of a randomized Hadamard
transform from its own stream ``default_rng([seed, 0x5167])``.

The pages measure on trained LLaMA/Qwen weights and WikiText-2/C4 text; the
synthetic tensors stand in for those, shaped like the projections the pages
name and carrying the outlier structure the pages describe (channel-wise
outliers, spikes about 1000x the normal values).

Draw order per workload: X base, outlier channels, spike positions, W.  The
Givens plan of group ``gamma`` comes from its own stream
``default_rng([seed, gamma])``: permutation of the pair list, then the
angles of every slot, then the 128 log-scales of the group's channels.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

GROUP = 128

__all__ = [
    "GROUP",
    "Workload",
    "WORKLOADS",
    "make",
    "round_to_bf16",
    "bf16_bits",
    "greedy_pair_plan",
    "givens_plan",
    "outlier_activations",
    "random_signs",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Direct rounding from float64, so there is no double rounding through
    float32: normal values keep 8 significant bits; below 2^-126 the grid is
    the subnormal spacing 2^-133.  Inputs must lie below the bf16 maximum.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def bf16_bits(x_bf16_valued: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float64 values that are exactly bf16-representable."""
    f = np.asarray(x_bf16_valued, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def outlier_activations(rng: np.random.Generator, M: int, K: int, n_channels: int = 8,
                        channel_gain: float = 100.0, spike_frac: float = 1e-4,
                        spike_gain: float = 1000.0) -> np.ndarray:
    """N(0,1) activations with channel-wise outliers and isolated spikes (float64)."""
    x = rng.standard_normal((M, K))
    ch = rng.choice(K, size=min(n_channels, K), replace=False)
    x[:, ch] *= channel_gain
    n_spikes = int(round(spike_frac * M * K))
    if n_spikes > 0:
        flat = rng.choice(M * K, size=n_spikes, replace=False)
        x.reshape(-1)[flat] *= spike_gain
    return x


def greedy_pair_plan(rng: np.random.Generator, g: int = GROUP, layers: int = 8,
                     per_layer: int = 64) -> list[list[tuple[int, int]]]:
    """Greedy selection of disjoint channel pairs for independent rotations.

    Follows the pair-selection procedure of the ParoQuant-style independent
    rotation article (codearts.csdn.net, section 2.2, "algorithm A1"): all
    pairs i < j of the g channels are put in one random order; each layer
    scans that order and keeps a pair when neither channel is already taken
    in this layer and the pair was not used by an earlier layer, stopping
    at ``per_layer`` pairs.  A layer may end with fewer pairs when the scan
    is exhausted.
    """
    all_pairs = [(i, j) for i in range(g) for j in range(i + 1, g)]
    order = rng.permutation(len(all_pairs))
    used = set()
    plan = []
    for _ in range(layers):
        taken = [False] * g
        chosen = []
        for idx in order:
            if len(chosen) >= per_layer:
                break
            i, j = all_pairs[idx]
            if taken[i] or taken[j] or (i, j) in used:
                continue
            chosen.append((i, j))
            taken[i] = taken[j] = True
        used.update(chosen)
        plan.append(chosen)
    return plan


def givens_plan(seed: int, K: int, layers: int = 8, per_layer: int = 64,
                theta_range: float = math.pi, beta_std: float = 0.1):
    """Rotation plan + angles + channel log-scales for every 128-channel group.

    Returns ``(pairs, theta, beta)``:
      pairs  uint8 [G, layers, per_layer, 2]; 0xFF marks an empty slot
      theta  float32 [G, layers, per_layer]; theta ~ U[-theta_range, theta_range]
      beta   float32 [K]; beta ~ N(0, beta_std)
    The float32 values are the inputs both sides use.
    """
    G = K // GROUP
    pairs = np.full((G, layers, per_layer, 2), 0xFF, dtype=np.uint8)
    theta = np.zeros((G, layers, per_layer), dtype=np.float32)
    beta = np.zeros((K,), dtype=np.float32)
    for gamma in range(G):
        rng = np.random.default_rng([seed, gamma])
        plan = greedy_pair_plan(rng, GROUP, layers, per_layer)
        for l, layer in enumerate(plan):
            for s, (i, j) in enumerate(layer):
                pairs[gamma, l, s, 0] = i
                pairs[gamma, l, s, 1] = j
        theta[gamma] = rng.uniform(-theta_range, theta_range,
                                   size=(layers, per_layer)).astype(np.float32)
        beta[gamma * GROUP:(gamma + 1) * GROUP] = rng.normal(0.0, beta_std,
                                                            size=GROUP).astype(np.float32)
    return pairs, theta, beta


def random_signs(seed: int, K: int) -> np.ndarray:
    """K independent signs, +1 or -1 with probability 1/2 (int8)."""
    rng = np.random.default_rng([seed, 0x5167])
    return np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)


@dataclass
class Workload:
    """One seeded synthetic workload.

    ``x`` holds the exact activation values (float64) the kernels receive;
    ``x_dtype`` says how they are stored ("f32" or "bf16").  ``w`` is the
    float32 weight in [K, N] layout.  ``transform`` is ("hadamard", block) or
    ("givens", layers); ``mode`` is "group128" or "rrs".
    """
    name: str
    M: int
    K: int
    N: int
    x: np.ndarray
    x_dtype: str
    w: np.ndarray
    transform: tuple
    mode: str
    y_dtype: str
    pairs: Optional[np.ndarray] = None
    theta: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    signs: Optional[np.ndarray] = None   # randomized Hadamard diagonal (int8 +-1)
    meta: dict = field(default_factory=dict)

    def x_storage(self) -> np.ndarray:
        """Activations in their storage form: float32 array, or uint16 bf16 bits."""
        if self.x_dtype == "f32":
            return self.x.astype(np.float32)
        return bf16_bits(self.x)


def _tiny(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    M, K, N = kw.get("M", 16), 128, 128
    x = rng.standard_normal((M, K))
    x[:, 5] *= 50.0
    x = x.astype(np.float32).astype(np.float64)
    w = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    return Workload("tiny", M, K, N, x, "f32", w, ("hadamard", 128), "group128", "f32")


def _q_proj(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    M, K, N = kw.get("M", 2048), kw.get("K", 4096), kw.get("N", 4096)
    x = round_to_bf16(outlier_activations(rng, M, K))
    w = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    return Workload("q_proj", M, K, N, x, "bf16", w, ("hadamard", 128), "group128", "bf16")


def _decode(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    M, K, N = kw.get("M", 16), kw.get("K", 4096), kw.get("N", 4096)
    layers = kw.get("layers", 8)
    x = round_to_bf16(outlier_activations(rng, M, K))
    w = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    pairs, theta, beta = givens_plan(seed, K, layers=layers)
    return Workload("decode", M, K, N, x, "bf16", w, ("givens", layers), "group128", "bf16",
                    pairs=pairs, theta=theta, beta=beta)


def _down_proj(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    M, K, N = kw.get("M", 4096), kw.get("K", 14336), kw.get("N", 4096)
    x = rng.standard_normal((M, K))
    n_heavy = int(round(0.001 * K))
    ch = rng.choice(K, size=n_heavy, replace=False)
    x[:, ch] = rng.standard_t(2.0, size=(M, n_heavy))
    x = round_to_bf16(x)
    w = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    return Workload("down_proj", M, K, N, x, "bf16", w, ("hadamard", 128), "group128", "bf16",
                    meta={"heavy_channels": np.sort(ch)})


def _rrs(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    M, K, N = kw.get("M", 8192), kw.get("K", 4096), kw.get("N", 11008)
    x = round_to_bf16(outlier_activations(rng, M, K))
    w = rng.normal(0.0, 0.02, size=(K, N)).astype(np.float32)
    return Workload("rrs", M, K, N, x, "bf16", w, ("hadamard", K), "rrs", "bf16")


def _kv(seed: int, **kw) -> Workload:
    rng = np.random.default_rng(seed)
    M, K = kw.get("M", 4096), kw.get("K", 1024)
    x = round_to_bf16(outlier_activations(rng, M, K))
    w = np.zeros((K, 0), dtype=np.float32)
    return Workload("kv", M, K, 0, x, "bf16", w, ("hadamard", 128), "group128", "bf16")


WORKLOADS = {
    "tiny": _tiny,
    "q_proj": _q_proj,
    "decode": _decode,
    "down_proj": _down_proj,
    "rrs": _rrs,
    "kv": _kv,
}


def make(name: str, seed: int = 0, signed: bool = False, **overrides) -> Workload:
    """Build workload ``name`` with ``seed``; overrides (M, K, N, layers) shrink it for tests.

    ``signed`` turns a Hadamard workload into its randomized form (a +-1
    diagonal from ``random_signs(seed, K)`` before each block)."""
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    wl = WORKLOADS[name](seed, **overrides)
    if signed:
        if wl.transform[0] != "hadamard":
            raise ValueError("signs apply to Hadamard transforms only")
        wl.signs = random_signs(seed, wl.K)
    return wl
