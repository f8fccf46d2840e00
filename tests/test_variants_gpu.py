"""GPU parity of the transform / quantizer variants: randomized (signed)
Hadamard transforms and dequantization (the INT4 KV-cache read-back),
through the C ABI against the CPU oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402
import oracle  # noqa: E402
from tests.helpers import case_seed, compare_codes, rel_fro, spec_of  # noqa: E402

if torch.cuda.is_available():
    import rotated_w4a4_amd as rw4  # noqa: E402
    from tests import gpu_util as gu  # noqa: E402
    from tests import test_parity_gpu as tp  # noqa: E402


SIGNED = [
    # name, M, K, N, block, mode, x dtype
    ("signed_h128", 300, 384, 200, 128, "group128", "bf16"),
    ("signed_h128_f32", 45, 1024, 64, 128, "group128", "f32"),
    ("signed_h512", 70, 1024, 96, 512, "group128", "bf16"),
    ("signed_h4096_rrs", 33, 4096, 80, 4096, "rrs", "bf16"),
]


@pytest.mark.parametrize("case", SIGNED, ids=[c[0] for c in SIGNED])
def test_signed_hadamard(case):
    name, M, K, N, b, mode, xdt = case
    rng = np.random.default_rng(case_seed(name))
    x = datagen.outlier_activations(rng, M, K)
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    wl = datagen.Workload(name, M, K, N, x, xdt, w, ("hadamard", b), mode, "f32",
                          signs=datagen.random_signs(11, K))
    t, xd, qa, sa, aref = tp._quant_parity(wl)
    qw, sw, wref = tp._weight_parity(wl, t)
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


def test_signs_change_codes_and_match_plain_when_all_positive():
    K, M = 256, 16
    rng = np.random.default_rng(12)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(gu.DEV)
    plain = rw4.Transform.hadamard(K, 128)
    ones = rw4.Transform.hadamard(K, 128, signs=np.ones(K, dtype=np.int8))
    signed = rw4.Transform.hadamard(K, 128, signs=datagen.random_signs(1, K))
    q0, s0 = rw4.quantize_act(plain, x)
    q1, s1 = rw4.quantize_act(ones, x)
    q2, _ = rw4.quantize_act(signed, x)
    torch.cuda.synchronize()
    assert torch.equal(q0, q1) and torch.equal(s0, s1)
    assert not torch.equal(q0, q2)


@pytest.mark.parametrize("shape", [(1, 128), (37, 384), (300, 1024)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_exact(shape, out):
    """dequantize of random stored codes and scales equals the oracle's product,
    rounded once to fp32 (then to bf16), bit for bit."""
    M, K = shape
    rng = np.random.default_rng(M * 7 + K)
    codes = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    scales = rng.uniform(1e-3, 10.0, size=(M, K // 128)).astype(np.float32)
    scales[0, 0] = 0.0
    q = torch.from_numpy(oracle.pack_int4(codes)).to(gu.DEV)
    s = torch.from_numpy(scales).to(gu.DEV)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = gu.to_np(rw4.dequantize(q, s, dt))
    ref = oracle.round_dequant_output(oracle.dequantize(codes, scales), out)
    assert np.array_equal(y, ref)


def test_dequantize_strided_output():
    M, K = 20, 256
    rng = np.random.default_rng(3)
    codes = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    scales = rng.uniform(0.1, 1.0, size=(M, 2)).astype(np.float32)
    q = torch.from_numpy(oracle.pack_int4(codes)).to(gu.DEV)
    s = torch.from_numpy(scales).to(gu.DEV)
    big = torch.full((M, K + 64), 7.0, dtype=torch.float32, device=gu.DEV)
    rw4.dequantize(q, s, out=big[:, :K])
    y = gu.to_np(big)
    assert np.array_equal(y[:, :K], oracle.round_dequant_output(oracle.dequantize(codes, scales), "f32"))
    assert np.all(y[:, K:] == 7.0)   # the padding beyond K is untouched


def test_kv_cache_roundtrip_full_size():
    """The INT4 KV-cache workload at its full size (4096 tokens x 8 heads x 128):
    quantize (block-128 Hadamard per head, group-128 INT4) and dequantize."""
    wl = datagen.make("kv")
    t, xd, qa, sa, aref = tp._quant_parity(wl)
    y = gu.to_np(rw4.dequantize(qa, sa, torch.bfloat16))
    # exact given the GPU's own codes and scales
    ref = oracle.round_dequant_output(oracle.dequantize(tp._unpack(qa), gu.to_np(sa)), "bf16")
    assert np.array_equal(y, ref)
    # and close to the transformed activations: RTN error within half a step
    xt = oracle.transform_act(wl.x, spec_of(wl))
    step = np.repeat(aref["sa"], 128, axis=1)
    assert np.all(np.abs(y - xt) <= step / 2 * (1 + 1e-2) + np.abs(xt) * 2 ** -8)
    print(f"kv: rel-Frobenius reconstruction error {rel_fro(y, xt):.3e}", flush=True)


def test_signed_weight_layouts_agree():
    rng = np.random.default_rng(8)
    K, N = 1024, 72
    w = torch.from_numpy(rng.normal(0, 0.02, size=(K, N)).astype(np.float32)).to(gu.DEV)
    sg = datagen.random_signs(4, K)
    for b in (128, 1024):
        t = rw4.Transform.hadamard(K, b, signs=sg)
        qw1, sw1 = rw4.pack_weight(t, w, "kn")
        qw2, sw2 = rw4.pack_weight(t, w.t().contiguous(), "nk")
        torch.cuda.synchronize()
        assert torch.equal(qw1, qw2) and torch.equal(sw1, sw2)


@pytest.mark.parametrize("layers", [4, 12, 16])
def test_givens_layer_counts(layers):
    """ParoQuant-style plans with other numbers of rotation layers (the plan is
    an input; the kernel batches its table loads 8 layers at a time)."""
    M, K, N = 6, 512, 40
    rng = np.random.default_rng(100 + layers)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, M, K))
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    plan = dict(zip(("pairs", "theta", "beta"), datagen.givens_plan(9, K, layers=layers)))
    wl = datagen.Workload(f"givens_L{layers}", M, K, N, x, "bf16", w, ("givens", layers), "group128", "f32",
                          **plan)
    t, xd, qa, sa, aref = tp._quant_parity(wl)
    qw, sw, wref = tp._weight_parity(wl, t)
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


# ---------------------------------------------------------------------------
# Quantization group sizes 64 and 256 (block-128 Hadamard)
# ---------------------------------------------------------------------------

def _group_quant_parity(x64, xdt, K, group, signs=None):
    spec = {"kind": "hadamard", "block": 128}
    if signs is not None:
        spec["signs"] = signs
    t = rw4.Transform.hadamard(K, 128, signs=signs)
    x = gu.x_to_device(x64, xdt)
    qa, sa = rw4.quantize_act(t, x, "group128", group=group)
    ref = oracle.quantize_act(x64, spec, "group128", group)
    tp._check_quant(tp._unpack(qa), gu.to_np(sa), ref["codes"], ref["ratio"], ref["sa"], f"act g{group}")
    return t, spec, qa, sa, ref


@pytest.mark.parametrize("M", [1100, 300, 7])  # 1100: the tiled kernel; 300 and 7: the small-M kernel
@pytest.mark.parametrize("signed", [False, True])
def test_group256_end_to_end(M, signed):
    K, N = 1024, 200
    rng = np.random.default_rng(31 + M)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, M, K))
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    signs = datagen.random_signs(5, K) if signed else None
    t, spec, qa, sa, aref = _group_quant_parity(x, "bf16", K, 256, signs)
    qw, sw = rw4.pack_weight(t, torch.from_numpy(w).to(gu.DEV), "kn", group=256)
    wref = oracle.pack_weight(w, spec, 256)
    tp._check_quant(tp._unpack(qw), gu.to_np(sw), wref["codes"], wref["ratio"], wref["sw"], "weight g256")
    assert sa.shape == (M, K // 256) and sw.shape == (N, K // 256)
    wl = datagen.Workload(f"g256_m{M}", M, K, N, x, "bf16", w, ("hadamard", 128), "group128", "f32")
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


@pytest.mark.parametrize("M", [300, 9])
def test_group256_accumulators_exact(M):
    """Group isolation at g = 256: sa = 1 and sw one-hot in group j give
    Y = acc[:, :, j] exactly (integers up to 256 * 49, exact in fp32)."""
    K, N = 1024, 144
    rng = np.random.default_rng(40 + M)
    ca = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    cw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    ca[0, :256], cw[0, :256] = 7, 7          # the extreme accumulator 256 * 49
    ca[1, 256:512], cw[0, 256:512] = -7, 7   # and its negative
    qa = torch.from_numpy(oracle.pack_int4(ca)).to(gu.DEV)
    qw = torch.from_numpy(oracle.pack_int4(cw)).to(gu.DEV)
    acc = oracle.group_accumulators(ca, cw, 256)
    sa = torch.ones((M, K // 256), dtype=torch.float32, device=gu.DEV)
    for j in range(K // 256):
        swn = np.zeros((N, K // 256), dtype=np.float32)
        swn[:, j] = 1.0
        y = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, torch.from_numpy(swn).to(gu.DEV), torch.float32))
        assert np.array_equal(y, acc[:, :, j].astype(np.float64)), f"group {j}"


def test_group64_quantize_dequantize():
    """A 64-group INT4 KV cache: quantize_act at g = 64, read back exactly."""
    M, K = 257, 1024
    rng = np.random.default_rng(50)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, M, K))
    t, spec, qa, sa, ref = _group_quant_parity(x, "bf16", K, 64)
    assert sa.shape == (M, K // 64)
    y = gu.to_np(rw4.dequantize(qa, sa, torch.float32))
    exact = oracle.round_dequant_output(oracle.dequantize(tp._unpack(qa), gu.to_np(sa), 64), "f32")
    assert np.array_equal(y, exact)
    step = np.repeat(ref["sa"], 64, axis=1)
    assert np.all(np.abs(y - ref["xt"]) <= step / 2 * (1 + 1e-2) + np.abs(ref["xt"]) * 2 ** -20)


def test_group64_fp32_ragged_groups():
    M, K = 33, 384                      # 6 groups of 64, a ragged quad of 128-blocks
    rng = np.random.default_rng(51)
    x = datagen.outlier_activations(rng, M, K).astype(np.float32).astype(np.float64)
    _group_quant_parity(x, "f32", K, 64)


def test_givens_fp16_angles():
    """Angles stored in half precision: the same transform as the fp32 entry
    point given the widened angles (identical codes), and oracle parity with
    the half-precision angles."""
    M, K, N = 40, 512, 48
    rng = np.random.default_rng(60)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, M, K))
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    pairs, theta, beta = datagen.givens_plan(13, K, layers=8)
    th16 = theta.astype(np.float16)
    t16 = rw4.Transform.givens(K, pairs, th16, beta)
    t32 = rw4.Transform.givens(K, pairs, th16.astype(np.float32), beta)
    xd = gu.x_to_device(x, "bf16")
    q16, s16 = rw4.quantize_act(t16, xd)
    q32, s32 = rw4.quantize_act(t32, xd)
    torch.cuda.synchronize()
    assert torch.equal(q16, q32) and torch.equal(s16, s32)
    wl = datagen.Workload("givens_f16", M, K, N, x, "bf16", w, ("givens", 8), "group128", "f32",
                          pairs=pairs, theta=th16, beta=beta)
    t, _, qa, sa, aref = tp._quant_parity(wl)
    qw, sw, wref = tp._weight_parity(wl, t)
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


@pytest.mark.parametrize("M", [1100, 300, 7])  # 1100: the tiled kernel; 300 and 7: the small-M kernel
def test_group64_end_to_end(M):
    """64-wide groups (the article's choice for outlier-heavy layers) through
    the GEMM: both kernels (large M and decode-sized M)."""
    K, N = 1024, 136
    rng = np.random.default_rng(70 + M)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, M, K))
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    t, spec, qa, sa, aref = _group_quant_parity(x, "bf16", K, 64)
    qw, sw = rw4.pack_weight(t, torch.from_numpy(w).to(gu.DEV), "kn", group=64)
    wref = oracle.pack_weight(w, spec, 64)
    tp._check_quant(tp._unpack(qw), gu.to_np(sw), wref["codes"], wref["ratio"], wref["sw"], "weight g64")
    wl = datagen.Workload(f"g64_m{M}", M, K, N, x, "bf16", w, ("hadamard", 128), "group128", "f32")
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


@pytest.mark.parametrize("M", [200, 5])
def test_group64_accumulators_exact(M):
    """Group isolation at g = 64 on both kernels: Y = acc[:, :, j] exactly."""
    K, N = 512, 72
    rng = np.random.default_rng(80 + M)
    ca = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    cw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    ca[0, 64:128], cw[1, 64:128] = -7, -7     # 64 * 49 in the odd half of a 128-group
    qa = torch.from_numpy(oracle.pack_int4(ca)).to(gu.DEV)
    qw = torch.from_numpy(oracle.pack_int4(cw)).to(gu.DEV)
    acc = oracle.group_accumulators(ca, cw, 64)
    sa = torch.ones((M, K // 64), dtype=torch.float32, device=gu.DEV)
    for j in range(K // 64):
        swn = np.zeros((N, K // 64), dtype=np.float32)
        swn[:, j] = 1.0
        y = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, torch.from_numpy(swn).to(gu.DEV), torch.float32))
        assert np.array_equal(y, acc[:, :, j].astype(np.float64)), f"group {j}"


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_extreme_scales(out):
    """Scales from subnormal to near the fp32 maximum, on both sides of the
    2^119 bound where the widened-FP8 path hands over to the per-code path:
    the product is still the exact c * s rounded once."""
    M, K = 6, 256
    rng = np.random.default_rng(90)
    codes = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    scales = np.array([[1e-45, 3e-39], [2.0 ** -126, 1.0], [2.0 ** 118, 2.0 ** 119],
                       [1e36, 4e37], [0.0, 7.5e-3], [2.0 ** 119 * 0.999, 3.3e38 / 7]], dtype=np.float32)
    q = torch.from_numpy(oracle.pack_int4(codes)).to(gu.DEV)
    s = torch.from_numpy(scales).to(gu.DEV)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = gu.to_np(rw4.dequantize(q, s, dt))
    ref = oracle.round_dequant_output(oracle.dequantize(codes, scales.astype(np.float64)), out)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("case", [("h128", 128, "group128", "bf16"), ("h128", 128, "group128", "f32"),
                                  ("rrs2048", 2048, "rrs", "bf16"), ("rrs2048", 2048, "rrs", "f32")],
                         ids=lambda c: f"{c[0]}-{c[3]}")
def test_strided_activations_and_output(case):
    """Activations as a column slice of a wider tensor (ldx > K) and the GEMM
    writing into a column slice of a wider output (ldy > N): same results as
    the contiguous calls, and the padding untouched."""
    name, block, mode, xdt = case
    M, K, N = 37, 2048, 40
    rng = np.random.default_rng(101)
    x = datagen.outlier_activations(rng, M, K)
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    t = rw4.Transform.hadamard(K, block)
    xd = gu.x_to_device(x, xdt)
    wide = torch.zeros((M, K + 96), dtype=xd.dtype, device=gu.DEV)
    wide[:, 32:32 + K] = xd
    qa0, sa0 = rw4.quantize_act(t, xd, mode)
    qa1, sa1 = rw4.quantize_act(t, wide[:, 32:32 + K], mode)
    qw, sw = rw4.pack_weight(t, torch.from_numpy(w).to(gu.DEV))
    y0 = rw4.w4a4_gemm(qa0, sa0, qw, sw, torch.bfloat16)
    ybig = torch.full((M, N + 24), 5.0, dtype=torch.bfloat16, device=gu.DEV)
    rw4.w4a4_gemm(qa0, sa0, qw, sw, out=ybig[:, 8:8 + N])
    torch.cuda.synchronize()
    assert torch.equal(qa0, qa1) and torch.equal(sa0, sa1)
    assert torch.equal(y0, ybig[:, 8:8 + N])
    assert torch.all(ybig[:, :8] == 5.0) and torch.all(ybig[:, 8 + N:] == 5.0)


@pytest.mark.parametrize("g", [64, 128, 256])
@pytest.mark.parametrize("M", [17, 32, 33, 50, 64, 65])
def test_small_batch_accumulators_exact(M, g):
    """Small batches (the small-M kernel with 2 or 4 row tiles up to M = 64,
    two 64-row chunks at M = 65): exact integer group sums by group
    isolation, with extreme accumulators in the last rows."""
    K, N = 512, 40
    rng = np.random.default_rng(1000 + M + g)
    ca = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    cw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    ca[M - 1, :g], cw[N - 1, :g] = 7, -7            # -g * 49 in the last row and column
    qa = torch.from_numpy(oracle.pack_int4(ca)).to(gu.DEV)
    qw = torch.from_numpy(oracle.pack_int4(cw)).to(gu.DEV)
    acc = oracle.group_accumulators(ca, cw, g)
    sa = torch.ones((M, K // g), dtype=torch.float32, device=gu.DEV)
    for j in (0, K // g - 1):
        swn = np.zeros((N, K // g), dtype=np.float32)
        swn[:, j] = 1.0
        y = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, torch.from_numpy(swn).to(gu.DEV), torch.float32))
        assert np.array_equal(y, acc[:, :, j].astype(np.float64)), f"M {M} g {g} group {j}"


@pytest.mark.parametrize("M", [24, 48, 64])
def test_small_batch_end_to_end(M):
    wl = datagen.make("decode", M=M, K=1024, N=256)
    t, xd, qa, sa, aref = tp._quant_parity(wl)
    qw, sw, wref = tp._weight_parity(wl, t)
    tp._gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


SMALL_ITER = [
    # M, g, K, N, scale columns to isolate: several K iterations (odd counts, a partial last
    # one) for 16-, 32- and 64-row tiles and every group size; 32-channel blocks (M <= 16,
    # N > 12288) with a partial last block
    (16, 128, 14336, 64, (0, 15, 16, 111)),
    (5, 64, 2176, 48, (0, 31, 32, 33)),
    (16, 256, 4352, 40, (0, 7, 8, 16)),
    (30, 128, 2176, 33, (0, 15, 16)),
    (64, 128, 1152, 24, (0, 7, 8)),
    (40, 256, 2304, 20, (0, 7, 8)),
    (64, 64, 1152, 17, (0, 15, 16, 17)),
    (3, 128, 256, 12304, (0, 1)),
    (16, 64, 512, 12296, (0, 7)),
    (16, 128, 4352, 12304, (0, 15, 16, 33)),
    # batches above 64 rows with few output tiles: 64-row chunks of A in one launch
    (100, 128, 2176, 40, (0, 15, 16)),
    (257, 64, 1152, 24, (0, 15, 16, 17)),
    (1000, 256, 512, 48, (0, 1)),
]

TILED_EDGES = [
    # M, g, K, N: products the tiled kernel takes (M > 1024, or a tiled grid of >= 128
    # blocks), with partial tiles on both edges and unaligned output rows
    (1100, 64, 384, 200),
    (1030, 256, 512, 129),
    (300, 128, 256, 5499),
]


@pytest.mark.parametrize("case", TILED_EDGES, ids=[f"M{c[0]}_g{c[1]}_K{c[2]}_N{c[3]}" for c in TILED_EDGES])
def test_tiled_kernel_edges_exact(case):
    """Exact integer group sums through the tiled kernel at ragged shapes (group
    isolation: sa = 1, sw one-hot on the first and the last scale column)."""
    M, g, K, N = case
    print(f"tiled edges M={M} g={g} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M + g + K + N)
    ca = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    cw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    ca[M - 1, :g], cw[N - 1, :g] = 7, -7
    qa = torch.from_numpy(oracle.pack_int4(ca)).to(gu.DEV)
    qw = torch.from_numpy(oracle.pack_int4(cw)).to(gu.DEV)
    acc = oracle.group_accumulators(ca, cw, g)
    G = K // g
    sa = torch.ones((M, G), dtype=torch.float32, device=gu.DEV)
    for j in (0, G - 1):
        swn = np.zeros((N, G), dtype=np.float32)
        swn[:, j] = 1.0
        y = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, torch.from_numpy(swn).to(gu.DEV), torch.float32))
        assert np.array_equal(y, acc[:, :, j].astype(np.float64)), f"M {M} g {g} K {K} N {N} column {j}"


@pytest.mark.parametrize("case", SMALL_ITER, ids=[f"M{c[0]}_g{c[1]}_K{c[2]}_N{c[3]}" for c in SMALL_ITER])
def test_small_batch_iterations_exact(case):
    """The small-M kernel over several K iterations, with 32-channel blocks and over
    64-row chunks of A:
    with sa = 1 and sw one-hot on scale column j, Y is the exact integer
    group sum of column j (fp32 output), for columns on both sides of the
    iteration boundaries."""
    M, g, K, N, cols = case
    print(f"small-M iterations M={M} g={g} K={K} N={N}", flush=True)
    rng = np.random.default_rng(M * 7 + g + K + N)
    ca = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    cw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    ca[M - 1, K - g:], cw[N - 1, K - g:] = -7, 7     # -g * 49 in the last group of the last row and column
    qa = torch.from_numpy(oracle.pack_int4(ca)).to(gu.DEV)
    qw = torch.from_numpy(oracle.pack_int4(cw)).to(gu.DEV)
    acc = oracle.group_accumulators(ca, cw, g)
    G = K // g
    sa = torch.ones((M, G), dtype=torch.float32, device=gu.DEV)
    for j in cols + (G - 1,):
        swn = np.zeros((N, G), dtype=np.float32)
        swn[:, j] = 1.0
        y = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, torch.from_numpy(swn).to(gu.DEV), torch.float32))
        assert np.array_equal(y, acc[:, :, j].astype(np.float64)), f"M {M} g {g} K {K} N {N} column {j}"


def test_many_rows_cross_the_grid_limit():
    """70 001 rows: the dequantize launcher splits rows into launches of at most
    65 535 (the grid's y limit), and the quantizer gives each wave several rows.
    Quantize against the oracle on rows around the split, dequantize exactly."""
    M, K = 70001, 256
    print(f"many rows M={M} K={K}", flush=True)
    rng = np.random.default_rng(70001)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, M, K))
    wl = datagen.Workload("many_rows", M, K, 0, x, "bf16", np.zeros((K, 0), np.float32), ("hadamard", 128),
                          "group128", "bf16")
    rows = np.r_[0:3, 65530:65540, M - 3:M]
    t, xd, qa, sa, ref = tp._quant_parity(wl, rows)
    codes = tp._unpack(qa).astype(np.float64)
    sa_np = gu.to_np(sa).astype(np.float64)
    got = gu.to_np(rw4.dequantize(qa, sa, torch.float32))
    want = (codes * np.repeat(sa_np, 128, axis=1)).astype(np.float32).astype(np.float64)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_tiled_kernel_strided_output(out):
    """The tiled kernel (M > 1024) writing into a column slice of a wider
    output (ldy > N, a row pitch that is not a multiple of 16 bytes, so the
    element-store path): the same values as the contiguous call, and the
    padding untouched."""
    M, K, N = 1100, 256, 200
    rng = np.random.default_rng(303)
    x = datagen.round_to_bf16(datagen.outlier_activations(rng, M, K))
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    t = rw4.Transform.hadamard(K, 128)
    qa, sa = rw4.quantize_act(t, gu.x_to_device(x, "bf16"))
    qw, sw = rw4.pack_weight(t, torch.from_numpy(w).to(gu.DEV))
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    y0 = rw4.w4a4_gemm(qa, sa, qw, sw, dt)
    c0 = 16 // wide_elem_bytes(dt)  # the output base must stay 16-byte aligned; its row pitch need not
    wide = torch.full((M, N + 27), 5.0, dtype=dt, device=gu.DEV)
    rw4.w4a4_gemm(qa, sa, qw, sw, out=wide[:, c0:c0 + N])
    torch.cuda.synchronize()
    assert torch.equal(y0, wide[:, c0:c0 + N])
    assert torch.all(wide[:, :c0] == 5.0) and torch.all(wide[:, c0 + N:] == 5.0)


def wide_elem_bytes(dt):
    return 2 if dt == torch.bfloat16 else 4
