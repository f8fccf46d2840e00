"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (from the method's parity contract):
  * INT4 codes equal except at rounding near-ties (|x/s - (k+1/2)| < 1e-4
    code units), where they may differ by exactly 1, at most 1e-4 of codes;
  * fp32 scales within 1e-5 relative;
  * int32 group accumulators bit-exact (group isolation: sa = 1, sw one-hot);
  * GEMM output from identical codes within 1e-5 relative (fp32 rounding of
    the epilogue), bf16 output within one bf16 ulp of the fp32 result;
  * end-to-end fp32 output within 2e-3 relative Frobenius of the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402
import oracle  # noqa: E402
from tests.helpers import (assert_gemm_close, case_seed, compare_codes, epilogue_error_bound,  # noqa: E402
                           rel_fro, spec_of)

if torch.cuda.is_available():
    import rotated_w4a4_amd as rw4  # noqa: E402
    from tests import gpu_util as gu  # noqa: E402


def _check_bytes(q_gpu, what):
    """The stored bytes are exactly the oracle's packing of the codes they hold
    (the paired form, zero with sign 0), byte for byte."""
    qb = gu.to_np(q_gpu)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(qb)), qb), f"{what}: stored bytes not canonical"


def _check_quant(codes_gpu, s_gpu, ref_codes, ref_ratio, ref_s, what):
    n, tot = compare_codes(codes_gpu, ref_codes, ref_ratio)
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    den = np.where(ref_s > 0, ref_s, 1.0)
    rel = np.abs(s_gpu - ref_s) / den
    assert np.all((ref_s > 0) | (s_gpu == 0)), f"{what}: zero scale mismatch"
    assert rel.max() <= 1e-5, f"{what}: scale rel err {rel.max():.3g}"
    print(f"{what}: {n}/{tot} near-tie code flips, max scale rel err {rel.max():.2e}", flush=True)


def _unpack(q):
    return oracle.unpack_int4(gu.to_np(q))


# ----------------------------------------------------------------------------
# Workload-level parity at full size
# ----------------------------------------------------------------------------

def _quant_parity(wl, rows=None):
    spec = spec_of(wl)
    t = gu.transform_for(wl)
    x = gu.x_to_device(wl.x, wl.x_dtype)
    qa, sa, ws = gu.quantize(t, x, wl.mode)
    _check_bytes(qa, f"{wl.name} act")
    ref = oracle.quantize_act(wl.x if rows is None or wl.mode == "rrs" else wl.x[rows], spec, wl.mode)
    codes = _unpack(qa)
    sa_np = gu.to_np(sa)
    rc, rr, rs = ref["codes"], ref["ratio"], ref["sa"]
    if rows is not None:
        codes, sa_np = codes[rows], sa_np[rows]
        if wl.mode == "rrs":
            rc, rr, rs = rc[rows], rr[rows], rs[rows]
    _check_quant(codes, sa_np, rc, rr, rs, f"{wl.name} act")
    if wl.mode == "rrs":
        s_gpu = gu.to_np(ws) / np.sqrt(int(wl.transform[1]))
        rel = np.abs(s_gpu - ref["s"]) / ref["s"]
        assert rel.max() <= 1e-5, rel.max()
    return t, x, qa, sa, ref


def _weight_parity(wl, t, cols=None):
    spec = spec_of(wl)
    w = torch.from_numpy(wl.w).to(gu.DEV)
    qw, sw = rw4.pack_weight(t, w, "kn")
    _check_bytes(qw, f"{wl.name} weight")
    wsel = wl.w if cols is None else wl.w[:, cols]
    ref = oracle.pack_weight(wsel, spec)
    codes = _unpack(qw)
    sw_np = gu.to_np(sw)
    if cols is not None:
        codes, sw_np = codes[cols], sw_np[cols]
    _check_quant(codes, sw_np, ref["codes"], ref["ratio"], ref["sw"], f"{wl.name} weight")
    return qw, sw, ref


def _gemm_parity(wl, qa, sa, qw, sw, rows, a_ref=None, w_ref=None, a_rows_in_ref=None, cols=None):
    """Y from identical codes (fp32 and bf16 outputs), then end-to-end vs the oracle's own codes.

    Identical codes: every compared output within 1e-5 of |y| plus the fp32
    summation bound of the epilogue (tests.helpers.epilogue_error_bound), and
    rel-Frobenius within 1e-5.  ``rows`` (and ``cols``) select the outputs
    compared; pass all rows to compare the whole output."""
    y32 = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, sw, torch.float32))
    y16 = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, sw, torch.bfloat16))
    cols = np.arange(y32.shape[1]) if cols is None else cols
    sel = np.ix_(rows, cols)
    qa_np, sa_np = gu.to_np(qa)[rows], gu.to_np(sa)[rows]
    qw_np, sw_np = gu.to_np(qw)[cols], gu.to_np(sw)[cols]
    y_ref = oracle.w4a4_gemm(qa_np, sa_np, qw_np, sw_np, "f64")
    g = 2 * qa_np.shape[1] // sa_np.shape[1]
    bound = epilogue_error_bound(oracle.unpack_int4(qa_np), sa_np, oracle.unpack_int4(qw_np), sw_np, g,
                                 oracle.group_accumulators)
    err, worst = assert_gemm_close(y32[sel], y_ref, bound, f"{wl.name}: GEMM from identical codes")
    # bf16 output: RNE of the fp32 result, within one bf16 ulp
    b = oracle.round_bf16(y32[sel])
    ulp = np.abs(b) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(y16[sel] - b) <= ulp), f"{wl.name}: bf16 output off by more than 1 ulp"
    if a_ref is not None:
        ar = a_ref if a_rows_in_ref is None else {k: (v[a_rows_in_ref] if k in ("qa", "sa") else v) for k, v in a_ref.items()}
        wq, wsc = (w_ref["qw"], w_ref["sw"])
        if len(wq) != len(cols):
            wq, wsc = wq[cols], wsc[cols]
        y_e2e = oracle.w4a4_gemm(ar["qa"], ar["sa"], wq, wsc, "f64")
        e2e = rel_fro(y32[sel], y_e2e)
        print(f"{wl.name}: {len(rows)}x{len(cols)} outputs, identical-codes rel {err:.2e} "
              f"(worst {worst:.2f} of the element bound), end-to-end rel-Frobenius {e2e:.2e}", flush=True)
        assert e2e <= 2e-3
    return y32


def test_tiny():
    wl = datagen.make("tiny")
    t, x, qa, sa, aref = _quant_parity(wl)
    qw, sw, wref = _weight_parity(wl, t)
    rows = np.arange(wl.M)
    _gemm_parity(wl, qa, sa, qw, sw, rows, aref, wref)


def test_q_proj_full():
    wl = datagen.make("q_proj")
    t, x, qa, sa, aref = _quant_parity(wl)
    qw, sw, wref = _weight_parity(wl, t)
    # the whole 2048 x 4096 output, element by element
    _gemm_parity(wl, qa, sa, qw, sw, np.arange(wl.M), aref, wref)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_givens(M):
    wl = datagen.make("decode", M=M)
    t, x, qa, sa, aref = _quant_parity(wl)
    qw, sw, wref = _weight_parity(wl, t)
    _gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


def test_down_proj_full():
    wl = datagen.make("down_proj")
    t, x, qa, sa, aref = _quant_parity(wl)
    qw, sw, wref = _weight_parity(wl, t)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(wl.M - 8, wl.M),
                                     np.random.default_rng(2).choice(wl.M, 240, replace=False)]))
    _gemm_parity(wl, qa, sa, qw, sw, rows, aref, wref, a_rows_in_ref=rows)


def test_down_proj_whole_output():
    """The whole 4096 x 4096 down_proj output from identical codes, element by
    element (the codes themselves are compared in test_down_proj_full), in
    row chunks so that the oracle's float64 products stay small."""
    wl = datagen.make("down_proj")
    t = gu.transform_for(wl)
    qa, sa, _ = gu.quantize(t, gu.x_to_device(wl.x, wl.x_dtype), wl.mode)
    qw, sw = rw4.pack_weight(t, torch.from_numpy(wl.w).to(gu.DEV), "kn")
    y32 = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, sw, torch.float32))
    qa_np, sa_np, qw_np, sw_np = gu.to_np(qa), gu.to_np(sa), gu.to_np(qw), gu.to_np(sw)
    ca_all, cw = oracle.unpack_int4(qa_np), oracle.unpack_int4(qw_np)
    worst = 0.0
    for r0 in range(0, wl.M, 512):
        rows = slice(r0, min(r0 + 512, wl.M))
        y_ref = oracle.w4a4_gemm(qa_np[rows], sa_np[rows], qw_np, sw_np, "f64")
        bound = epilogue_error_bound(ca_all[rows], sa_np[rows], cw, sw_np, 128, oracle.group_accumulators)
        _, w = assert_gemm_close(y32[rows], y_ref, bound, f"down_proj rows {r0}..: GEMM from identical codes")
        worst = max(worst, w)
        print(f"down_proj whole output: rows {r0}..{rows.stop} match (worst {w:.2f} of the element bound)",
              flush=True)
    print(f"down_proj whole output: {wl.M}x{wl.N} outputs, worst {worst:.2f} of the element bound", flush=True)


def test_rrs_full():
    wl = datagen.make("rrs")
    t, x, qa, sa, aref = _quant_parity(wl)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(wl.N - 16, wl.N),
                                     np.random.default_rng(3).choice(wl.N, 480, replace=False)]))
    qw, sw, wref = _weight_parity(wl, t, cols=cols)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(wl.M - 8, wl.M),
                                     np.random.default_rng(4).choice(wl.M, 240, replace=False)]))
    _gemm_parity(wl, qa, sa, qw, sw, rows, aref, wref, a_rows_in_ref=rows, cols=cols)


# ----------------------------------------------------------------------------
# int32 exactness: group isolation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2048, 4096, 4096), (16, 4096, 4096), (300, 1024, 200)])
def test_group_isolation_int32_exact(shape):
    M, K, N = shape
    G = K // 128
    rng = np.random.default_rng(M + N)
    ca = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    cw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    ca[0, :128] = -7
    cw[0, :128] = -7   # the extreme accumulator 128 * 49
    if N > 1:
        cw[1, :128] = 7  # and its negative
    qa = torch.from_numpy(oracle.pack_int4(ca)).to(gu.DEV)
    qw = torch.from_numpy(oracle.pack_int4(cw)).to(gu.DEV)
    sa = torch.ones((M, G), dtype=torch.float32, device=gu.DEV)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 24), replace=False)]))
    for g in sorted({0, G - 1, int(rng.integers(G))}):
        swn = np.zeros((N, G), dtype=np.float32)
        swn[:, g] = 1.0
        sw = torch.from_numpy(swn).to(gu.DEV)
        y = gu.to_np(rw4.w4a4_gemm(qa, sa, qw, sw, torch.float32))
        acc = oracle.group_accumulators(ca[rows][:, g * 128:(g + 1) * 128],
                                        cw[:, g * 128:(g + 1) * 128], 128)[:, :, 0]
        assert np.array_equal(y[rows].astype(np.int64), acc), f"group {g}"
        assert np.array_equal(y[rows], acc.astype(np.float64))
        if g == 0:
            assert y[0, 0] == 6272.0
            if N > 1:
                assert y[0, 1] == -6272.0


# ----------------------------------------------------------------------------
# Ragged shapes, every transform, edge inputs
# ----------------------------------------------------------------------------

RAGGED = [
    # name, M, K, N, transform, mode, x dtype
    ("h128_ragged", 300, 384, 200, ("hadamard", 128), "group128", "bf16"),
    ("h128_f32", 77, 640, 48, ("hadamard", 128), "group128", "f32"),
    ("h128_m1", 1, 256, 33, ("hadamard", 128), "group128", "bf16"),
    ("h256_full_rows", 130, 1024, 64, ("hadamard", 256), "group128", "bf16"),
    ("h1024_rrs", 97, 1024, 144, ("hadamard", 1024), "rrs", "bf16"),
    ("h128_rrs", 50, 512, 16, ("hadamard", 128), "rrs", "f32"),
    ("h8192_rrs", 20, 8192, 32, ("hadamard", 8192), "rrs", "bf16"),
    ("h2048_rrs_f32", 37, 2048, 40, ("hadamard", 2048), "rrs", "f32"),
    ("h4096_rrs_ragged", 130, 4096, 24, ("hadamard", 4096), "rrs", "bf16"),
    ("h4096_rrs_f32", 9, 4096, 16, ("hadamard", 4096), "rrs", "f32"),
    ("givens_prefill", 70, 512, 96, ("givens", 3), "group128", "bf16"),
    ("givens_f32", 5, 256, 17, ("givens", 8), "group128", "f32"),
    # batches the tiled kernel takes (M > 1024, or a tiled grid of >= 128 blocks), partial
    # tiles on both edges and output rows that break 16-byte alignment; the cases above with
    # 64 < M <= 1024 and few output tiles run on the small-M kernel in 64-row chunks
    ("h128_tiled_m1100", 1100, 256, 72, ("hadamard", 128), "group128", "bf16"),
    ("h128_tiled_wide", 200, 256, 16257, ("hadamard", 128), "group128", "bf16"),
    ("givens_tiled_m1030", 1030, 256, 131, ("givens", 8), "group128", "bf16"),
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_ragged(case):
    name, M, K, N, tr, mode, xdt = case
    rng = np.random.default_rng(case_seed(name))
    x = datagen.outlier_activations(rng, M, K)
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    kw = {}
    if tr[0] == "givens":
        kw = dict(zip(("pairs", "theta", "beta"), datagen.givens_plan(7, K, layers=tr[1])))
    wl = datagen.Workload(name, M, K, N, x, xdt, w, tr, mode, "f32", **kw)
    t, xd, qa, sa, aref = _quant_parity(wl)
    qw, sw, wref = _weight_parity(wl, t)
    _gemm_parity(wl, qa, sa, qw, sw, np.arange(M), aref, wref)


def test_weight_layouts_agree():
    """pack_weight of W [K, N] and of its [N, K] transpose give identical bytes."""
    rng = np.random.default_rng(5)
    K, N = 512, 96
    w = torch.from_numpy(rng.normal(0, 0.02, size=(K, N)).astype(np.float32)).to(gu.DEV)
    for t in (rw4.Transform.hadamard(K, 128), rw4.Transform.hadamard(K, 512)):
        qw1, sw1 = rw4.pack_weight(t, w, "kn")
        qw2, sw2 = rw4.pack_weight(t, w.t().contiguous(), "nk")
        torch.cuda.synchronize()
        assert torch.equal(qw1, qw2) and torch.equal(sw1, sw2)


def test_edge_inputs():
    """All-zero rows/groups, constant rows, a huge spike, subnormals, bf16 extremes."""
    K, M = 512, 8
    x = np.zeros((M, K))
    x[1] = 3.0                                  # constant row
    x[2, 5] = 3.0e4                             # one huge spike
    x[3, :128] = 1e-39                          # fp32 subnormals (bf16 keeps them)
    x[4] = np.tile([1.0, -1.0], K // 2)         # +-1 pattern
    x[5, 200] = -3.3e38                         # near the bf16 maximum
    x[6, 300:302] = [2.0 ** -20, -(2.0 ** -20)]
    x = datagen.round_to_bf16(x)
    wl = datagen.Workload("edge", M, K, 8, x, "bf16", np.zeros((K, 8), np.float32),
                          ("hadamard", 128), "group128", "f32")
    t, xd, qa, sa, aref = _quant_parity(wl)
    codes = _unpack(qa)
    assert not codes[0].any() and not gu.to_np(sa)[0].any()      # zero row -> zero codes and scales
    assert not codes[7].any()


def test_zero_weights_and_empty_calls():
    t = rw4.Transform.hadamard(256, 128)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=gu.DEV)
    qa, sa = rw4.quantize_act(t, x)
    assert qa.shape == (0, 128)
    y = rw4.w4a4_gemm(qa, sa, torch.zeros((5, 128), dtype=torch.uint8, device=gu.DEV),
                      torch.zeros((5, 2), device=gu.DEV), torch.float32)
    assert y.shape == (0, 5)
    w = torch.zeros((256, 4), device=gu.DEV)
    qw, sw = rw4.pack_weight(t, w)
    torch.cuda.synchronize()
    assert not qw.any() and not sw.any()


@pytest.mark.parametrize("shape", [(512, 4096, 1024), (2048, 1024, 1024), (16, 4096, 12304)],
                         ids=["small_kernel_chunks", "tiled_kernel", "small_kernel_32ch"])
def test_bitwise_determinism(shape):
    M, K, N = shape
    wl = datagen.make("q_proj", M=M, K=K, N=N)
    t = gu.transform_for(wl)
    x = gu.x_to_device(wl.x, wl.x_dtype)
    w = torch.from_numpy(wl.w).to(gu.DEV)
    outs = []
    for _ in range(3):
        qa, sa = rw4.quantize_act(t, x)
        qw, sw = rw4.pack_weight(t, w)
        y = rw4.w4a4_gemm(qa, sa, qw, sw, torch.bfloat16)
        torch.cuda.synchronize()
        outs.append((qa.clone(), sa.clone(), qw.clone(), sw.clone(), y.clone()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)
