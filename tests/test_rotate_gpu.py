"""GPU parity of rotate_act (the transform alone, unquantized) and the INT4
KV-cache attention scores it exists for: keys stored rotated and quantized
(quantize_act), read back (dequantize), queries rotated alike (rotate_act);
(q R)(k R)^T = q k^T because R is orthogonal (the OstQuant page, section 3.2,
rotates queries and keys together; the Rotated Runtime Smooth experiments
quantize the KV cache in groups of 128).

Bars, derived from the fp32 arithmetic of the kernels (u = 2^-24):
  * Hadamard blocks of b: each of the log2(b) butterfly stages and the two
    scalings round once, so |x~_gpu - x~| <= (log2 b + 2) u sum_j |x_j| / sqrt(b);
  * Givens: every layer rotates pairs with fp32 cos/sin (rounded from f64),
    so the group's error norm is at most (4.3 L + 2) u ||x_g||_2 max(alpha^-1);
  * bf16 outputs: additionally within half a bf16 step (2^-8 relative) of the value.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402
import oracle  # noqa: E402
from tests.helpers import case_seed, rel_fro, spec_of  # noqa: E402

if torch.cuda.is_available():
    import rotated_w4a4_amd as rw4  # noqa: E402
    from tests import gpu_util as gu  # noqa: E402

U = 2.0 ** -24


def _bound(x, spec):
    """Element-wise bound on the fp32 transform's rounding error (see the module docstring)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    M, K = x.shape
    if spec["kind"] == "hadamard":
        b = int(spec["block"])
        s = x.reshape(M, K // b, b).sum(axis=2) / math.sqrt(b)
        return np.repeat(s, b, axis=1) * (math.log2(b) + 2) * U
    L = spec["pairs"].shape[1]
    ainv = np.exp(-spec["beta"].astype(np.float64)).reshape(K // 128, 128).max(axis=1)
    n = np.sqrt((x.reshape(M, K // 128, 128) ** 2).sum(axis=2)) * ainv[None, :]
    return np.repeat(n, 128, axis=1) * (4.3 * L + 2) * U


CASES = [
    # name, M, K, transform, signed, x dtype
    ("h128_bf16", 300, 1024, ("hadamard", 128), False, "bf16"),
    ("h128_f32_m1", 1, 256, ("hadamard", 128), False, "f32"),
    ("h128_signed", 77, 640, ("hadamard", 128), True, "bf16"),
    ("h1024_rows", 50, 2048, ("hadamard", 1024), False, "bf16"),
    ("h4096_full", 33, 4096, ("hadamard", 4096), True, "f32"),
    ("givens8", 40, 512, ("givens", 8), False, "bf16"),
    ("givens3_f32", 5, 256, ("givens", 3), False, "f32"),
]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rotate_act_parity(case, out):
    name, M, K, tr, signed, xdt = case
    rng = np.random.default_rng(case_seed(name))
    x = datagen.outlier_activations(rng, M, K)
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    kw = {}
    if tr[0] == "givens":
        kw = dict(zip(("pairs", "theta", "beta"), datagen.givens_plan(5, K, layers=tr[1])))
    wl = datagen.Workload(name, M, K, 0, x, xdt, np.zeros((K, 0), np.float32), tr, "group128", "f32",
                          signs=datagen.random_signs(3, K) if signed else None, **kw)
    spec = spec_of(wl)
    t = gu.transform_for(wl)
    xd = gu.x_to_device(x, xdt)
    y = gu.to_np(rw4.rotate_act(t, xd, torch.float32 if out == "f32" else torch.bfloat16))
    ref = oracle.transform_act(x, spec)
    bound = _bound(x, spec)
    if out == "bf16":
        bound = bound * (1 + 2.0 ** -8) + np.abs(ref) * 2.0 ** -8
    d = np.abs(y - ref)
    assert np.all(d <= bound), f"{name}: worst excess {(d - bound).max():.3g}"
    print(f"{name} {out}: max |err| / bound {float((d / np.maximum(bound, 1e-300)).max()):.3f}", flush=True)


def test_rotate_act_strided_and_empty():
    K, M = 256, 9
    t = rw4.Transform.hadamard(K, 128)
    rng = np.random.default_rng(1)
    x = datagen.round_to_bf16(rng.standard_normal((M, K)))
    big = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=gu.DEV)
    big[:, :K] = gu.x_to_device(x, "bf16")
    out = torch.full((M, K + 32), 5.0, dtype=torch.float32, device=gu.DEV)
    rw4.rotate_act(t, big[:, :K], out=out[:, :K])
    y = gu.to_np(out)
    assert np.all(y[:, K:] == 5.0)  # padding untouched
    ref = oracle.transform_act(x, {"kind": "hadamard", "block": 128})
    assert np.all(np.abs(y[:, :K] - ref) <= _bound(x, {"kind": "hadamard", "block": 128}))
    e = rw4.rotate_act(t, torch.zeros((0, K), dtype=torch.bfloat16, device=gu.DEV))
    assert e.shape == (0, K)


def test_kv_attention_scores_full_size():
    """The INT4 KV-cache workload at full size (4096 tokens x 8 heads x 128):
    keys through quantize_act + dequantize, queries through rotate_act; the
    scores (q R)(k_hat R)^T per head against the oracle's, on 256 query rows
    x all 4096 keys x 8 heads.  Bound per score: each rotated query value is
    within 2^-8 + 9u of its exact value (bf16 output), each key value exact
    up to one fp32 rounding, so |dS| <= (2^-8 + 12 u) sum_d |q~_d| |k~_d|."""
    kv = datagen.make("kv")              # keys
    qw = datagen.make("kv", seed=1)      # queries of the same shape and recipe
    M, K, H = kv.M, kv.K, kv.K // 128
    spec = spec_of(kv)
    t = gu.transform_for(kv)
    qk, sk = rw4.quantize_act(t, gu.x_to_device(kv.x, "bf16"))
    khat = gu.to_np(rw4.dequantize(qk, sk, torch.float32))          # k_hat R (rotated domain)
    qr = gu.to_np(rw4.rotate_act(t, gu.x_to_device(qw.x, "bf16")))  # q R, bf16
    rows = np.random.default_rng(7).choice(M, 256, replace=False)
    # oracle: exact rotation of the queries; the keys from the GPU's own codes and scales
    qr_ref = oracle.transform_act(qw.x[rows], spec)
    k_ref = oracle.dequantize(oracle.unpack_int4(gu.to_np(qk)), gu.to_np(sk))
    worst = 0.0
    errs_rot, errs_plain = [], []
    for h in range(H):
        sl = slice(128 * h, 128 * (h + 1))
        s_gpu = qr[rows][:, sl] @ khat[:, sl].T
        s_ref = qr_ref[:, sl] @ k_ref[:, sl].T
        bound = (2.0 ** -8 + 12 * U) * (np.abs(qr_ref[:, sl]) @ np.abs(k_ref[:, sl]).T)
        d = np.abs(s_gpu - s_ref)
        assert np.all(d <= bound), f"head {h}: worst excess {(d - bound).max():.3g}"
        worst = max(worst, float((d / np.maximum(bound, 1e-300)).max()))
        # what the rotation buys: scores against the unquantized keys, versus INT4
        # keys quantized without the rotation (oracle, same group-128 RTN)
        s_true = qw.x[rows][:, sl] @ kv.x[:, sl].T
        errs_rot.append(rel_fro(s_gpu, s_true))
        kq, ks, _ = oracle.quantize_groups(kv.x[:, sl])
        errs_plain.append(rel_fro(qw.x[rows][:, sl] @ oracle.dequantize(kq, ks).T, s_true))
    print(f"kv scores: worst |dS| / bound {worst:.3f}; rel-Frobenius vs unquantized keys "
          f"{np.mean(errs_rot):.3e} rotated INT4, {np.mean(errs_plain):.3e} unrotated INT4", flush=True)
    assert np.mean(errs_rot) < np.mean(errs_plain)
