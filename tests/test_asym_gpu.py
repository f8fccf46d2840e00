"""GPU parity of the asymmetric (s, z) path: quantize_act_asym, the weight code
sums, w4a4_gemm_asym and dequantize_asym, against the oracle.

[Paro] (the independent rotation article) section 2.3: a 128-channel group
shares (s, z); the Rotated Runtime Smooth symbol table: q = round(x * scale)
+ offset.  Bars:
  * codes: the centred codes q - z equal the oracle's except at rounding
    near-ties (of x / s, or of -lo / s, which moves z and the clamped
    minimum by one), at most 1e-4 of them; scales within 1e-6 relative;
    zero points equal except at near-ties of -lo / s;
  * code sums: exact;
  * GEMM from identical codes: element-wise within 1e-5 |y| plus the fp32
    epilogue bound over the centred accumulators (tests.helpers), bf16
    within one ulp of the rounded fp32 result; end to end (the oracle's own
    codes) rel-Frobenius <= 2e-3;
  * dequantize_asym: exactly the fp32 (then bf16) rounding of s (q - z).
Shapes cover the small-M kernel (M <= 1024 with few tiles) and the tiled one
(2048 x 4096 x 4096, the whole output), ragged N, f32 and bf16 inputs,
random signs, and inputs with a per-row offset (a DC component that the
block Hadamard turns into one large channel per block, the case the zero
point is for).
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
    # name, M, K, N, signed, x dtype, per-row offset
    ("asym_small_m5", 5, 1024, 300, False, "bf16", True),
    ("asym_m1_f32", 1, 256, 17, False, "f32", True),
    ("asym_signed_m77", 77, 640, 96, True, "bf16", False),
    ("asym_mid_m300", 300, 1024, 1000, False, "bf16", True),
    ("asym_decode16_k14336", 16, 14336, 512, False, "bf16", True),
    ("asym_q_proj_full", 2048, 4096, 4096, False, "bf16", True),
]


def _inputs(name, M, K, N, xdt, offset):
    rng = np.random.default_rng(case_seed(name))
    x = datagen.outlier_activations(rng, M, K)
    if offset:
        x = x + rng.uniform(0.5, 3.0, size=(M, 1))
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    return x, w


def _check_asym_codes(u_gpu, s_gpu, z_gpu, ref, what):
    g = 128
    R, K = u_gpu.shape
    zr = np.repeat(ref["za"], g, axis=1)
    zg = np.repeat(z_gpu.astype(np.int64), g, axis=1)
    c_gpu = u_gpu.astype(np.int64) - zg
    c_ref = ref["codes"].astype(np.int64) - zr
    near = (tie_distance(ref["ratio"]) < 1e-4) | np.repeat(tie_distance(ref["zratio"]) < 1e-4, g, axis=1)
    diff = c_gpu != c_ref
    assert np.all(np.abs(c_gpu - c_ref) <= 1), f"{what}: a centred code off by more than one"
    assert not (diff & ~near).any(), f"{what}: {int((diff & ~near).sum())} code differences away from ties"
    assert diff.sum() <= int(np.floor(1e-4 * diff.size)), f"{what}: {int(diff.sum())} near-tie flips"
    zdiff = z_gpu.astype(np.int64) != ref["za"]
    assert not (zdiff & ~(tie_distance(ref["zratio"]) < 1e-4)).any(), f"{what}: zero points differ"
    live = ref["sa"] > 0
    rel = np.abs(s_gpu[live] - ref["sa"][live]) / ref["sa"][live]
    assert rel.max(initial=0) <= 1e-6, f"{what}: scale rel err {rel.max():.3g}"
    assert not s_gpu[~live].any() and not z_gpu[~live].any()
    print(f"{what}: {int(diff.sum())}/{diff.size} near-tie flips, {int(zdiff.sum())} zero-point flips, "
          f"max scale rel err {rel.max(initial=0):.2e}", flush=True)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_asym_path(case):
    name, M, K, N, signed, xdt, offset = case
    print(f"{name}: M={M} K={K} N={N}", flush=True)
    x, w = _inputs(name, M, K, N, xdt, offset)
    signs = datagen.random_signs(case_seed(name) % 89, K) if signed else None
    spec = {"kind": "hadamard", "block": 128, "signs": signs}
    t = rw4.Transform.hadamard(K, 128, signs=signs)
    xd = gu.x_to_device(x, xdt)
    qa, sa, za = rw4.quantize_act_asym(t, xd)
    u = oracle.unpack_uint4(gu.to_np(qa))
    assert np.array_equal(oracle.pack_uint4(u), gu.to_np(qa))  # the stored bytes are the oracle's packing
    sa_np, za_np = gu.to_np(sa), gu.to_np(za)
    assert np.array_equal(za_np, np.rint(za_np)) and za_np.min() >= 0 and za_np.max() <= 15
    ref = oracle.quantize_act(x, spec, "group128_asym")
    _check_asym_codes(u, sa_np, za_np, ref, f"{name} act")

    # weights: the symmetric pack, then their code sums
    qw, sw = rw4.pack_weight(t, torch.from_numpy(w).to(gu.DEV), "kn")
    cw = rw4.weight_code_sums(qw)
    qw_np, sw_np = gu.to_np(qw), gu.to_np(sw)
    assert np.array_equal(gu.to_np(cw), oracle.weight_code_sums(qw_np).astype(np.float64))

    # the GEMM from identical codes, element by element over the whole output
    y32 = gu.to_np(rw4.w4a4_gemm_asym(qa, sa, za, qw, sw, cw, torch.float32))
    y16 = gu.to_np(rw4.w4a4_gemm_asym(qa, sa, za, qw, sw, cw, torch.bfloat16))
    qa_np = gu.to_np(qa)
    y_ref = oracle.w4a4_gemm_asym(qa_np, sa_np, za_np.astype(np.int64), qw_np, sw_np, "f64")
    centred = u.astype(np.int64) - np.repeat(za_np.astype(np.int64), 128, axis=1)
    bound = epilogue_error_bound(centred, sa_np, oracle.unpack_int4(qw_np), sw_np, 128, oracle.group_accumulators)
    err, worst = assert_gemm_close(y32, y_ref, bound, f"{name}: asym GEMM from identical codes")
    b = oracle.round_bf16(y32)
    assert np.all(np.abs(y16 - b) <= np.abs(b) * 2.0 ** -7 + 1e-30), f"{name}: bf16 output off by more than 1 ulp"
    # end to end against the oracle's own codes and weights
    wref = oracle.pack_weight(w, spec)
    y_e2e = oracle.w4a4_gemm_asym(ref["qa"], ref["sa"], ref["za"], wref["qw"], wref["sw"], "f64")
    e2e = rel_fro(y32, y_e2e)
    print(f"{name}: identical-codes rel {err:.2e} (worst {worst:.2f} of the element bound), end-to-end "
          f"rel-Frobenius {e2e:.2e}", flush=True)
    assert e2e <= 2e-3

    # dequantize: exactly the rounded s (q - z)
    if M * K <= 4 * 2 ** 20:
        for dt, name_ in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            xh = gu.to_np(rw4.dequantize_asym(qa, sa, za, dt))
            expect = oracle.round_dequant_output(oracle.dequantize_asym(u, sa_np, za_np), name_)
            assert np.array_equal(xh, expect), f"{name}: dequantize_asym {name_}"


def test_asym_beats_symmetric_on_offset_rows():
    """With a per-row offset the block Hadamard concentrates it in one channel per
    block, so a group's values are one-sided around a large value: the zero
    point halves the step, and the layer's error against the exact X W drops."""
    name, M, K, N = "asym_vs_sym", 256, 4096, 512
    x, w = _inputs(name, M, K, N, "bf16", True)
    t = rw4.Transform.hadamard(K, 128)
    xd = gu.x_to_device(x, "bf16")
    qw, sw = rw4.pack_weight(t, torch.from_numpy(w).to(gu.DEV), "kn")
    cw = rw4.weight_code_sums(qw)
    qa, sa, za = rw4.quantize_act_asym(t, xd)
    y_asym = gu.to_np(rw4.w4a4_gemm_asym(qa, sa, za, qw, sw, cw, torch.float32))
    qs, ss = rw4.quantize_act(t, xd)
    y_sym = gu.to_np(rw4.w4a4_gemm(qs, ss, qw, sw, torch.float32))
    exact = x @ w.astype(np.float64)
    ea, es = rel_fro(y_asym, exact), rel_fro(y_sym, exact)
    print(f"{name}: rel-Frobenius vs exact X W: asymmetric {ea:.4e}, symmetric {es:.4e}", flush=True)
    assert ea < es


def test_asym_empty_and_unsupported():
    t = rw4.Transform.hadamard(256, 128)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=gu.DEV)
    qa, sa, za = rw4.quantize_act_asym(t, x)
    assert qa.shape == (0, 128) and sa.shape == (0, 2) and za.shape == (0, 2)
    t512 = rw4.Transform.hadamard(512, 512)
    with pytest.raises(rw4.RW4Error, match="UNSUPPORTED"):
        rw4.quantize_act_asym(t512, torch.zeros((2, 512), dtype=torch.bfloat16, device=gu.DEV))
    # a row of zeros: scale and zero point 0, codes 0
    z = torch.zeros((3, 256), dtype=torch.float32, device=gu.DEV)
    z[1, :] = 1.0
    qa, sa, za = rw4.quantize_act_asym(t, z)
    assert not gu.to_np(qa)[0].any() and not gu.to_np(sa)[0].any() and not gu.to_np(za)[0].any()
