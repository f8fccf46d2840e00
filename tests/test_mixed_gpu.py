"""GPU parity of the 8-bit groups for extreme outliers (the independent
rotation article, section 4.1: mixed precision): quantize_act_mixed,
extend_weight_groups and the INT4 GEMM over the extended K, against the
oracle.

Bars: the two planes of the GPU (unpacked h, l) rebuild q8 = 15 h + l, and
q8 and the INT4 codes equal the oracle's except at rounding near-ties of
x / scale (at most 1e-4 of the codes, each off by one); scales within 1e-6
relative; the extended weights are an exact copy; the GEMM from identical
codes element-wise within the fp32 epilogue bound (tests.helpers) over the
extended K, and end to end (the oracle's own codes) within 2e-3
rel-Frobenius.  Inputs carry a few extreme outlier channels; the named
groups are the ones holding them.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402
import oracle  # noqa: E402
from tests.helpers import assert_gemm_close, case_seed, epilogue_error_bound, rel_fro, tie_distance  # noqa: E402

if torch.cuda.is_available():
    import rotated_w4a4_amd as rw4  # noqa: E402
    from tests import gpu_util as gu  # noqa: E402

CASES = [
    # name, M, K, N, 8-bit groups, x dtype, signed
    ("mixed_small", 7, 512, 96, [3, 1], "bf16", False),
    ("mixed_m1_f32", 1, 256, 40, [0], "f32", False),
    ("mixed_signed", 300, 1024, 200, [5], "bf16", True),
    ("mixed_none", 33, 384, 64, [], "bf16", False),
    ("mixed_q_proj", 2048, 4096, 4096, [4, 17, 30], "bf16", False),
    # 11 groups (a partial last quad), four 8-bit groups, three of them in one quad
    ("mixed_dense_quad", 65, 1408, 48, [8, 9, 10, 2], "f32", True),
]


def _inputs(name, M, K, N, groups8, xdt):
    rng = np.random.default_rng(case_seed(name))
    x = datagen.outlier_activations(rng, M, K)
    for g in groups8:  # an extreme channel in every named group
        x[:, g * 128 + 5] *= 400.0
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    return x, w


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mixed_path(case):
    name, M, K, N, groups8, xdt, signed = case
    print(f"{name}: M={M} K={K} N={N} 8-bit groups {groups8}", flush=True)
    x, w = _inputs(name, M, K, N, groups8, xdt)
    G, n8 = K // 128, len(groups8)
    signs = datagen.random_signs(case_seed(name) % 83, K) if signed else None
    spec = {"kind": "hadamard", "block": 128, "signs": signs}
    t = rw4.Transform.hadamard(K, 128, signs=signs)
    slot, glist = rw4.mixed_tables(K, groups8, gu.DEV)
    xd = gu.x_to_device(x, xdt)
    qa, sa = rw4.quantize_act_mixed(t, xd, slot, n8)
    planes = oracle.unpack_int4(gu.to_np(qa)).astype(np.int64)
    assert np.array_equal(oracle.pack_int4(planes), gu.to_np(qa))  # both planes in the canonical stored form
    sa_np = gu.to_np(sa)
    ref = oracle.quantize_act(x, spec, "group128_mixed", order=groups8)
    # rebuild the one-code form from the planes
    q = planes[:, :K].copy()
    for j, g in enumerate(groups8):
        sl = slice(g * 128, (g + 1) * 128)
        q[:, sl] = 15 * planes[:, sl] + planes[:, K + j * 128:K + (j + 1) * 128]
    diff = q != ref["codes"]
    assert np.all(np.abs(q - ref["codes"]) <= 1)
    assert not (diff & (tie_distance(ref["ratio"]) >= 1e-4)).any(), f"{name}: code differences away from ties"
    assert diff.sum() <= int(np.floor(1e-4 * diff.size)), f"{name}: {int(diff.sum())} near-tie flips"
    live = ref["sa"] > 0
    rel = np.abs(sa_np[live] - ref["sa"][live]) / ref["sa"][live]
    assert rel.max(initial=0) <= 1e-6, f"{name}: scale rel err {rel.max():.3g}"
    # each h plane's codes in [-7, 7] and the plane scales 15 s8 and s8
    for j, g in enumerate(groups8):
        np.testing.assert_allclose(sa_np[:, G + j] * 15.0, sa_np[:, g], rtol=1e-6)
    print(f"{name} act: {int(diff.sum())}/{diff.size} near-tie flips, max scale rel err {rel.max(initial=0):.2e}",
          flush=True)

    qw, sw = rw4.pack_weight(t, torch.from_numpy(w).to(gu.DEV), "kn")
    qx, sx = rw4.extend_weight_groups(qw, sw, glist)
    qw_np, sw_np = gu.to_np(qw), gu.to_np(sw)
    cx_ref, sx_ref = oracle.extend_weight_groups(oracle.unpack_int4(qw_np), sw_np, groups8)
    assert np.array_equal(oracle.unpack_int4(gu.to_np(qx)), cx_ref) and np.array_equal(gu.to_np(sx), sx_ref)

    y32 = gu.to_np(rw4.w4a4_gemm(qa, sa, qx, sx, torch.float32))
    y_ref = oracle.w4a4_gemm(gu.to_np(qa), sa_np, gu.to_np(qx), gu.to_np(sx), "f64")
    bound = epilogue_error_bound(planes, sa_np, cx_ref, sx_ref, 128, oracle.group_accumulators)
    err, worst = assert_gemm_close(y32, y_ref, bound, f"{name}: GEMM over the extended K")
    wref = oracle.pack_weight(w, spec)
    y_def = oracle.mixed_gemm_reference(ref["codes"], ref["scales"], groups8, wref["codes"], wref["sw"])
    e2e = rel_fro(y32, y_def)
    exact = x @ w.astype(np.float64)
    y4 = gu.to_np(rw4.w4a4_gemm(*rw4.quantize_act(t, xd), qw, sw, torch.float32))
    print(f"{name}: identical-codes rel {err:.2e} (worst {worst:.2f} of the bound), end-to-end {e2e:.2e}; "
          f"vs exact X W: mixed {rel_fro(y32, exact):.4e}, all INT4 {rel_fro(y4, exact):.4e}", flush=True)
    assert e2e <= 2e-3
    if n8:
        assert rel_fro(y32, exact) < rel_fro(y4, exact)
