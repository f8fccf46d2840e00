"""GPU parity of Rotated Runtime Smooth with the channel reorder (the
Rotated Runtime Smooth page, Figure 4 (1)-(2)) through the C ABI.

The channel order is an integer decided by floating point (fp32 maxima on
the GPU, float64 in the oracle): the GPU's order must be a permutation whose
oracle maxima never increase by more than 1e-5 relative from one position to
the next (so it differs from the oracle's only among near-equal maxima), and
it is then given to the oracle as input for the code and scale parity
(the parity bars of the other quantizers).  Weight codes and their
permutation are exact."""
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


def _check_order(order_gpu, xt):
    order_ref, m = oracle.rrs_channel_order(xt)
    K = xt.shape[1]
    assert sorted(order_gpu.tolist()) == list(range(K)), "order is not a permutation"
    mm = m[order_gpu]
    assert np.all(mm[1:] <= mm[:-1] * (1 + 1e-5)), "order not decreasing in the channel maxima"
    return int((order_gpu != order_ref).sum())


def _run(name, x, xdt, K, block, signs, w, cols=None, rows=None):
    spec = {"kind": "hadamard", "block": block}
    if signs is not None:
        spec["signs"] = signs
    t = rw4.Transform.hadamard(K, block, signs=signs)
    xd = gu.x_to_device(x, xdt)
    qa, sa, order = rw4.quantize_act_rrs_reorder(t, xd)
    order_np = gu.to_np(order).astype(np.int64)
    xt = oracle.transform_act(x, spec)
    moved = _check_order(order_np, xt)
    ref = oracle.quantize_act(x, spec, "rrs_reorder", order=order_np)
    codes = oracle.unpack_int4(gu.to_np(qa))
    n, tot = compare_codes(codes, ref["codes"], ref["ratio"])
    sa_np = gu.to_np(sa)
    rel = np.abs(sa_np - ref["sa"]) / np.where(ref["sa"] > 0, ref["sa"], 1.0)
    assert np.all((ref["sa"] > 0) | (sa_np == 0)) and rel.max() <= 1e-5, rel.max()
    # weights: per-channel scales, then the codes permuted by the activations' order
    wd = torch.from_numpy(w).to(gu.DEV)
    qw, sw = rw4.pack_weight_per_channel(t, wd)
    cols = np.arange(w.shape[1]) if cols is None else cols
    wref = oracle.pack_weight(w[:, cols], spec, per_channel=True)
    wcodes = oracle.unpack_int4(gu.to_np(qw))[cols]
    compare_codes(wcodes, wref["codes"], wref["ratio"])
    sw_np = gu.to_np(sw)[cols]
    wrel = np.abs(sw_np - wref["sw"]) / np.where(wref["sw"] > 0, wref["sw"], 1.0)
    assert wrel.max() <= 1e-5, wrel.max()
    assert np.all(sw_np == sw_np[:, :1])  # one scale per output channel
    qw_ord = rw4.permute_codes(qw, order)
    qw_ord_np = gu.to_np(qw_ord)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(qw_ord_np)), qw_ord_np)  # permuted codes repacked canonically
    assert np.array_equal(oracle.unpack_int4(qw_ord_np), oracle.permute_codes(oracle.unpack_int4(gu.to_np(qw)), order_np))
    # the product: identical codes element-wise, then end to end
    y = gu.to_np(rw4.w4a4_gemm(qa, sa, qw_ord, sw, torch.float32))
    rows = np.arange(x.shape[0]) if rows is None else rows
    sel = np.ix_(rows, cols)
    qa_np = gu.to_np(qa)[rows]
    y_ref = oracle.w4a4_gemm(qa_np, sa_np[rows], qw_ord_np[cols], sw_np, "f64")
    bound = epilogue_error_bound(oracle.unpack_int4(qa_np), sa_np[rows], oracle.unpack_int4(qw_ord_np[cols]), sw_np,
                                 128, oracle.group_accumulators)
    err, worst = assert_gemm_close(y[sel], y_ref, bound, f"{name}: GEMM from identical codes")
    w_ord_ref = oracle.pack_int4(oracle.permute_codes(wref["codes"], order_np))
    y_e2e = oracle.w4a4_gemm(ref["qa"][rows], ref["sa"][rows], w_ord_ref, wref["sw"], "f64")
    e2e = rel_fro(y[sel], y_e2e)
    print(f"{name}: {moved} order positions differ from the oracle's (near-equal maxima); {n}/{tot} code flips; "
          f"identical-codes rel {err:.2e} (worst {worst:.2f} of bound); end-to-end {e2e:.2e}", flush=True)
    assert e2e <= 2e-3


def test_rrs_reorder_full_size():
    """The Rotated Runtime Smooth workload at full size: 8192 x 4096 activations,
    full-row Hadamard, weights 4096 x 11008 (oracle weights on 512 columns,
    outputs compared on 256 rows x those columns)."""
    wl = datagen.make("rrs")
    cols = np.unique(np.concatenate([np.arange(16), np.arange(wl.N - 16, wl.N),
                                     np.random.default_rng(3).choice(wl.N, 480, replace=False)]))
    rows = np.unique(np.concatenate([np.arange(8), np.arange(wl.M - 8, wl.M),
                                     np.random.default_rng(4).choice(wl.M, 240, replace=False)]))
    _run("rrs_reorder", wl.x, "bf16", wl.K, wl.K, None, wl.w, cols=cols, rows=rows)


CASES = [
    # name, M, K, block, signed, x dtype, N
    ("h512_bf16", 37, 512, 512, False, "bf16", 40),
    ("h128_signed_f32", 20, 1024, 128, True, "f32", 24),
    ("h1024_k2048", 130, 2048, 1024, False, "bf16", 72),
    ("h4096_m1", 1, 4096, 4096, False, "bf16", 16),
    # whole-row blocks of 2048 and 4096 take the register / DPP transform kernels
    ("h2048_full_f32", 70, 2048, 2048, False, "f32", 24),
    ("h4096_full_m300", 300, 4096, 4096, False, "bf16", 32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rrs_reorder_ragged(case):
    name, M, K, block, signed, xdt, N = case
    rng = np.random.default_rng(case_seed(name))
    x = datagen.outlier_activations(rng, M, K)
    x = datagen.round_to_bf16(x) if xdt == "bf16" else x.astype(np.float32).astype(np.float64)
    w = rng.normal(0, 0.02, size=(K, N)).astype(np.float32)
    _run(name, x, xdt, K, block, datagen.random_signs(2, K) if signed else None, w)


@pytest.mark.parametrize("rows,K", [(1, 128), (77, 512), (1500, 4096), (3, 8192)])
def test_permute_codes_exact(rows, K):
    rng = np.random.default_rng(rows + K)
    codes = rng.integers(-7, 8, size=(rows, K)).astype(np.int8)
    order = rng.permutation(K).astype(np.int32)
    q = torch.from_numpy(oracle.pack_int4(codes)).to(gu.DEV)
    out = gu.to_np(rw4.permute_codes(q, torch.from_numpy(order).to(gu.DEV)))
    assert np.array_equal(oracle.unpack_int4(out), oracle.permute_codes(codes, order))
