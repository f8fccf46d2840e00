"""GPU parity of decode_fused: one launch that quantizes a decode step's
activations inside the small-M GEMM (the independent-rotation article,
section 3.2, fuses rotation, scaling and quantization into one kernel; the
QuIP#/QTIP page, section 6.1, fuses against launch latency at batch 1).

The fused kernel uses the arithmetic of quantize_act and of the small-M
w4a4_gemm, so its output must be bit-identical to those two calls in a row
(both output dtypes); the two-call path is itself held to the oracle by the
parity tests, and the smaller cases here are also checked against the oracle
end to end (codes, then the product within the epilogue's fp32 bound).
Shapes cover one and several 16-slice iterations, a ragged last iteration
(K = 2176: 17 slices), a K below one iteration (K = 384 and 128), ragged N,
one, two and four passes of four rows, random signs, and both channel
tilings (16 and, past 12288 channels, 32 per block).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402
from tests.helpers import case_seed  # noqa: E402

if torch.cuda.is_available():
    import rotated_w4a4_amd as rw4  # noqa: E402
    from tests import gpu_util as gu  # noqa: E402
    from tests import test_parity_gpu as tp  # noqa: E402

CASES = [
    # name, M, K, N, transform, signed, x dtype, oracle end to end
    ("h128_m16_q", 16, 4096, 4096, ("hadamard", 128), False, "bf16", True),
    ("h128_m1_k384_f32", 1, 384, 100, ("hadamard", 128), False, "f32", True),
    ("h128_m7_ct2", 7, 256, 12320, ("hadamard", 128), False, "bf16", False),
    ("h128_m5_k2176", 5, 2176, 300, ("hadamard", 128), False, "bf16", True),
    ("h128_m4_signed", 4, 4096, 4096, ("hadamard", 128), True, "bf16", False),
    ("h128_signed_m16_ct2_f32", 16, 1024, 13000, ("hadamard", 128), True, "f32", False),
    ("h128_m1_k128", 1, 128, 17, ("hadamard", 128), False, "bf16", True),
    ("h128_m12_k14336_f32", 12, 14336, 96, ("hadamard", 128), False, "f32", False),
]


def _workload(case):
    name, M, K, N, tr, signed, xdt, _ = case
    rng = np.random.default_rng(case_seed(name))
    x = datagen.outlier_activations(rng, M, K)
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    kw = {}
    if tr[0] == "givens":
        kw = dict(zip(("pairs", "theta", "beta"), datagen.givens_plan(case_seed(name) % 1000, K, layers=tr[1])))
    return datagen.Workload(name, M, K, N, x, xdt, w, tr, "group128", "f32",
                            signs=datagen.random_signs(case_seed(name) % 97, K) if signed else None, **kw)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_fused_matches_two_calls(case):
    wl = _workload(case)
    print(f"{wl.name}: M={wl.M} K={wl.K} N={wl.N}", flush=True)
    if case[-1]:
        # the two-call path against the oracle first: codes, weights, product
        t, xd, qa, sa, aref = tp._quant_parity(wl)
        qw, sw, wref = tp._weight_parity(wl, t)
        tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(wl.M), aref, wref)
    else:
        t = gu.transform_for(wl)
        xd = gu.x_to_device(wl.x, wl.x_dtype)
        qa, sa = rw4.quantize_act(t, xd)
        qw, sw = rw4.pack_weight(t, torch.from_numpy(wl.w).to(gu.DEV), "kn")
    for dt in (torch.float32, torch.bfloat16):
        y2 = rw4.w4a4_gemm(qa, sa, qw, sw, dt)
        y1 = rw4.decode_fused(t, xd, qw, sw, dt)
        torch.cuda.synchronize()
        assert y1.dtype == dt and y1.shape == (wl.M, wl.N)
        diff = (y1.float() != y2.float()).sum().item()
        assert torch.equal(y1, y2), f"{wl.name} {dt}: {diff} outputs differ from quantize_act + w4a4_gemm"
    # twice in a row into the same output: nothing left over from the first call
    out = torch.full((wl.M, wl.N), float("nan"), dtype=torch.float32, device=gu.DEV)
    rw4.decode_fused(t, xd, qw, sw, out=out)
    rw4.decode_fused(t, xd, qw, sw, out=out)
    assert torch.equal(out, rw4.w4a4_gemm(qa, sa, qw, sw, torch.float32))


def test_decode_fused_strided_rows_and_limits():
    """Rows with a pitch above K, an output pitch above N, the empty step,
    and the refusals (17 rows, Hadamard blocks other than 128, Givens)."""
    wl = _workload(("h128_pitch", 9, 512, 64, ("hadamard", 128), False, "bf16", False))
    t = gu.transform_for(wl)
    xd = gu.x_to_device(wl.x, wl.x_dtype)
    wide = torch.zeros((wl.M, wl.K + 64), dtype=torch.bfloat16, device=gu.DEV)
    wide[:, : wl.K] = xd
    xs = wide[:, : wl.K]
    qw, sw = rw4.pack_weight(t, torch.from_numpy(wl.w).to(gu.DEV), "kn")
    qa, sa = rw4.quantize_act(t, xd)
    ref = rw4.w4a4_gemm(qa, sa, qw, sw, torch.float32)
    ybig = torch.zeros((wl.M, wl.N + 8), dtype=torch.float32, device=gu.DEV)
    rw4.decode_fused(t, xs, qw, sw, out=ybig[:, : wl.N])
    assert torch.equal(ybig[:, : wl.N], ref)
    assert torch.count_nonzero(ybig[:, wl.N:]) == 0
    empty = rw4.decode_fused(t, xd[:0], qw, sw, torch.float32)
    assert empty.shape == (0, wl.N)
    x17 = torch.zeros((17, wl.K), dtype=torch.bfloat16, device=gu.DEV)
    with pytest.raises(rw4.RW4Error, match="SHAPE"):
        rw4.decode_fused(t, x17, qw, sw)
    t256 = rw4.Transform.hadamard(wl.K, 256)
    with pytest.raises(rw4.RW4Error, match="UNSUPPORTED"):
        rw4.decode_fused(t256, xd, qw, sw)
    g8 = rw4.Transform.givens(wl.K, *datagen.givens_plan(9, wl.K, layers=8))
    with pytest.raises(rw4.RW4Error, match="UNSUPPORTED"):
        rw4.decode_fused(g8, xd, qw, sw)
