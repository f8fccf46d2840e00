"""C ABI: the library loads, exports every declared symbol, and rejects bad
arguments on the host before any device work (no compute calls here)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rw4.h")

rw4 = pytest.importorskip("rotated_w4a4_amd", reason="librw4.so not built")
lib = rw4.lib

OK, ARG, SHAPE, UNSUP, HIP, NOMEM = range(6)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rw4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_hot_calls():
    names = _declared_functions()
    for n in ("rw4_quantize_act", "rw4_pack_weight", "rw4_w4a4_gemm"):
        assert n in names


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(rw4.EXPORTED_SYMBOLS)


def test_status_strings_and_version():
    for s in range(6):
        assert lib.rw4_status_str(s).decode().startswith("RW4_")
    assert rw4.version() == "0.1.0"


def _had(K, block):
    h = ctypes.c_void_p()
    st = lib.rw4_transform_hadamard(K, block, None, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("K,block,expect", [
    (0, 128, SHAPE), (100, 128, SHAPE), (4096, 64, SHAPE), (4096, 96, SHAPE),
    (4096, 8192, SHAPE), (384, 256, SHAPE), (14336, 256, UNSUP), (4096, 128, OK),
    (4096, 4096, OK), (14336, 128, OK)])
def test_hadamard_transform_validation(K, block, expect):
    st, h = _had(K, block)
    assert st == expect
    if st == OK:
        assert lib.rw4_transform_k(h) == K
        assert lib.rw4_transform_destroy(h) == OK
    else:
        assert not h.value


def test_null_out_pointer():
    assert lib.rw4_transform_hadamard(4096, 128, None, None) == ARG


def _givens_tables(K=256, L=2):
    G = K // 128
    pairs = np.full((G, L, 64, 2), 0xFF, np.uint8)
    for g in range(G):
        for l in range(L):
            for s in range(60):
                pairs[g, l, s] = (2 * s + l % 2, 2 * s + 1 + l % 2) if 2 * s + 1 + l % 2 < 128 else (0xFF, 0xFF)
    return pairs, np.zeros((G, L, 64), np.float32), np.zeros(K, np.float32)


@pytest.mark.parametrize("bad", ["i_ge_j", "range", "reuse", "half_empty"])
def test_givens_rejects_bad_pair_tables(bad):
    pairs, theta, beta = _givens_tables()
    if bad == "i_ge_j":
        pairs[0, 0, 0] = (5, 5)
    elif bad == "range":
        pairs[1, 1, 3] = (3, 200)
    elif bad == "reuse":
        pairs[0, 1, 0] = (1, 9)
        pairs[0, 1, 1] = (9, 11)
    else:
        pairs[0, 0, 2] = (0xFF, 7)
    h = ctypes.c_void_p()
    st = lib.rw4_transform_givens(256, 2, pairs.ctypes.data, theta.ctypes.data, beta.ctypes.data,
                                  None, ctypes.byref(h))
    assert st == ARG and not h.value


def test_givens_shape_and_null_checks():
    pairs, theta, beta = _givens_tables()
    h = ctypes.c_void_p()
    assert lib.rw4_transform_givens(250, 2, pairs.ctypes.data, theta.ctypes.data, beta.ctypes.data, None, ctypes.byref(h)) == SHAPE
    assert lib.rw4_transform_givens(256, 0, pairs.ctypes.data, theta.ctypes.data, beta.ctypes.data, None, ctypes.byref(h)) == SHAPE
    assert lib.rw4_transform_givens(256, 2, None, theta.ctypes.data, beta.ctypes.data, None, ctypes.byref(h)) == ARG


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device error path")
def test_givens_without_device_reports_hip_error():
    pairs, theta, beta = _givens_tables()
    h = ctypes.c_void_p()
    st = lib.rw4_transform_givens(256, 2, pairs.ctypes.data, theta.ctypes.data, beta.ctypes.data,
                                  None, ctypes.byref(h))
    assert st in (HIP, NOMEM) and not h.value


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case below fails validation first


def test_quantize_act_validation():
    st, t = _had(4096, 128)
    assert st == OK
    q = lib.rw4_quantize_act
    # null transform, bad mode, bad dtype
    assert q(None, 0, FAKE, 1, 4, 4096, FAKE, FAKE, None, None) == ARG
    assert q(t, 7, FAKE, 1, 4, 4096, FAKE, FAKE, None, None) == ARG
    assert q(t, 0, FAKE, 9, 4, 4096, FAKE, FAKE, None, None) == ARG
    # M == 0 is a no-op even with null buffers; negative M is a shape error
    assert q(t, 0, None, 1, 0, 4096, None, None, None, None) == OK
    assert q(t, 0, FAKE, 1, -1, 4096, FAKE, FAKE, None, None) == SHAPE
    # null buffers, ld too small, misaligned pointers and pitch
    assert q(t, 0, None, 1, 4, 4096, FAKE, FAKE, None, None) == ARG
    assert q(t, 0, FAKE, 1, 4, 4095, FAKE, FAKE, None, None) == ARG
    assert q(t, 0, FAKE + 2, 1, 4, 4096, FAKE, FAKE, None, None) == ARG
    assert q(t, 0, FAKE, 1, 4, 4100, FAKE, FAKE, None, None) == ARG  # 8200-byte pitch
    assert q(t, 0, FAKE, 1, 4, 4096, FAKE + 4, FAKE, None, None) == ARG
    # RRS needs a workspace, and is unsupported for K outside the row-kernel set
    assert q(t, 1, FAKE, 1, 4, 4096, FAKE, FAKE, None, None) == ARG
    lib.rw4_transform_destroy(t)
    st, t2 = _had(14336, 128)
    assert q(t2, 1, FAKE, 1, 4, 14336, FAKE, FAKE, FAKE, None) == UNSUP
    lib.rw4_transform_destroy(t2)


def test_pack_weight_validation():
    st, t = _had(1024, 128)
    p = lib.rw4_pack_weight
    assert p(None, FAKE, 0, 8, 8, 1, FAKE, FAKE, None) == ARG
    assert p(t, FAKE, 3, 8, 8, 1, FAKE, FAKE, None) == ARG
    assert p(t, None, 0, 0, 8, 1, None, None, None) == OK
    assert p(t, FAKE, 0, -2, 8, 1, FAKE, FAKE, None) == SHAPE
    assert p(t, FAKE, 0, 8, 0, 1, FAKE, FAKE, None) == ARG
    assert p(t, FAKE + 2, 0, 8, 8, 1, FAKE, FAKE, None) == ARG
    assert p(t, FAKE, 0, 8, 8, 1, FAKE + 1, FAKE, None) == ARG
    lib.rw4_transform_destroy(t)


def test_gemm_validation():
    g = lib.rw4_w4a4_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 100, FAKE, 0, 4, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 0, FAKE, 0, 4, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 4, 128, FAKE, 0, 4, None) == SHAPE
    # K above 2^24 (the per-block buffer ranges) is a shape error
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, (1 << 24) + 128, FAKE, 0, 4, None) == SHAPE
    assert g(None, None, None, None, 0, 4, 128, None, 0, 4, None) == OK
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, 5, 4, None) == ARG
    assert g(None, FAKE, FAKE, FAKE, 4, 4, 128, FAKE, 0, 4, None) == ARG
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 8, 128, FAKE, 0, 4, None) == ARG
    assert g(FAKE, FAKE, FAKE + 8, FAKE, 4, 4, 128, FAKE, 0, 4, None) == ARG


def test_signed_hadamard_validation():
    import numpy as np
    h = ctypes.c_void_p()
    f = lib.rw4_transform_hadamard_signed
    good = np.ones(256, dtype=np.int8)
    bad = good.copy()
    bad[7] = 0
    assert f(256, 128, None, None, ctypes.byref(h)) == ARG
    assert f(256, 128, good.ctypes.data, None, None) == ARG
    assert f(256, 128, bad.ctypes.data, None, ctypes.byref(h)) == ARG
    assert f(100, 128, good.ctypes.data, None, ctypes.byref(h)) == SHAPE
    assert f(256, 96, good.ctypes.data, None, ctypes.byref(h)) == SHAPE


def test_dequantize_validation():
    d = lib.rw4_dequantize
    assert d(FAKE, FAKE, 4, 100, FAKE, 0, 100, None) == SHAPE
    assert d(FAKE, FAKE, -1, 128, FAKE, 0, 128, None) == SHAPE
    assert d(None, None, 0, 128, None, 0, 128, None) == OK
    assert d(FAKE, FAKE, 4, 128, FAKE, 7, 128, None) == ARG
    assert d(None, FAKE, 4, 128, FAKE, 0, 128, None) == ARG
    assert d(FAKE, FAKE, 4, 128, FAKE, 0, 64, None) == ARG
    assert d(FAKE, FAKE, 4, 128, FAKE + 4, 0, 128, None) == ARG
    assert d(FAKE, FAKE, 4, 128, FAKE, 1, 132, None) == ARG   # bf16 rows of 264 bytes: not 16-aligned



def _plain_hadamard(K, block):
    h = ctypes.c_void_p()
    assert lib.rw4_transform_hadamard(K, block, None, ctypes.byref(h)) == OK
    return h


def test_group_size_validation_quantize_and_pack():
    """Group sizes other than 64/128/256 are argument errors, a group that does
    not divide K is a shape error, and combinations without a kernel say so;
    all of it before any pointer is looked at or anything is launched."""
    q, p = lib.rw4_quantize_act_g, lib.rw4_pack_weight_g
    h128 = _plain_hadamard(512, 128)
    h512 = _plain_hadamard(512, 512)
    h384 = _plain_hadamard(384, 128)
    try:
        for g, expect in ((96, ARG), (0, ARG), (-128, ARG), (512, ARG)):
            assert q(h128, 0, g, FAKE, 1, 4, 512, FAKE, FAKE, None, None) == expect
            assert p(h128, g, FAKE, 0, 4, 4, 1, FAKE, FAKE, None) == expect
        assert q(h384, 0, 256, FAKE, 1, 4, 384, FAKE, FAKE, None, None) == SHAPE
        assert p(h384, 256, FAKE, 0, 4, 4, 1, FAKE, FAKE, None) == SHAPE
        assert q(h512, 0, 64, FAKE, 1, 4, 512, FAKE, FAKE, None, None) == UNSUP   # block 512
        assert q(h128, 1, 256, FAKE, 1, 4, 512, FAKE, FAKE, FAKE, None) == UNSUP  # RRS
        assert p(h512, 256, FAKE, 0, 4, 4, 1, FAKE, FAKE, None) == UNSUP
        assert p(h512, 64, FAKE, 0, 4, 4, 1, FAKE, FAKE, None) == UNSUP
        # supported combinations with nothing to do
        for g in (64, 128, 256):
            assert q(h128, 0, g, None, 1, 0, 512, None, None, None, None) == OK
        assert p(h128, 256, None, 0, 0, 4, 1, None, None, None) == OK
    finally:
        for h in (h128, h512, h384):
            lib.rw4_transform_destroy(h)


def test_group_size_validation_gemm_and_dequantize():
    gm, dq = lib.rw4_w4a4_gemm_g, lib.rw4_dequantize_g
    assert gm(FAKE, FAKE, FAKE, FAKE, 4, 4, 512, 96, FAKE, 0, 4, None) == ARG
    assert gm(FAKE, FAKE, FAKE, FAKE, 4, 4, 384, 256, FAKE, 0, 4, None) == SHAPE
    assert gm(FAKE, FAKE, FAKE, FAKE, 4, 4, 192, 64, FAKE, 0, 4, None) == SHAPE   # K % 128
    assert gm(None, None, None, None, 4, 0, 512, 64, None, 0, 4, None) == OK
    assert gm(None, None, None, None, 0, 4, 512, 256, None, 0, 4, None) == OK
    assert dq(FAKE, FAKE, 4, 512, 96, FAKE, 0, 512, None) == ARG
    assert dq(FAKE, FAKE, 4, 384, 256, FAKE, 0, 384, None) == SHAPE
    assert dq(FAKE, FAKE, 4, 192, 128, FAKE, 0, 192, None) == SHAPE
    assert dq(None, None, 0, 192, 64, None, 0, 192, None) == OK
    # the unsuffixed calls are the 128-group ones
    assert lib.rw4_dequantize(FAKE, FAKE, 4, 192, FAKE, 0, 192, None) == SHAPE


def test_givens_f16_validation():
    h = ctypes.c_void_p()
    g = lib.rw4_transform_givens_f16
    assert g(100, 8, FAKE, FAKE, FAKE, None, ctypes.byref(h)) == SHAPE
    assert g(128, 0, FAKE, FAKE, FAKE, None, ctypes.byref(h)) == SHAPE
    assert g(128, 8, FAKE, None, FAKE, None, ctypes.byref(h)) == ARG
    assert g(128, 8, FAKE, FAKE, FAKE, None, None) == ARG
    # a non-finite half angle is rejected before anything is uploaded
    theta = np.zeros((1, 1, 64), dtype=np.float16)
    theta[0, 0, 3] = np.inf
    pairs = np.full((1, 1, 64, 2), 0xFF, dtype=np.uint8)
    beta = np.zeros(128, dtype=np.float32)
    assert g(128, 1, pairs.ctypes.data, theta.ctypes.data, beta.ctypes.data, None, ctypes.byref(h)) == ARG
    assert not h.value


@pytest.mark.parametrize("where", ["theta_nan", "theta_inf", "beta_nan", "beta_overflow"])
def test_givens_f32_rejects_non_finite(where):
    """The fp32 entry point rejects what the fp16 one rejects: a non-finite
    angle of a used slot, or a channel scale exp(+-beta) that is not a finite
    nonzero fp32 value, before anything is uploaded."""
    pairs, theta, beta = _givens_tables(K=128, L=1)
    if where == "theta_nan":
        theta[0, 0, 2] = np.nan
    elif where == "theta_inf":
        theta[0, 0, 0] = -np.inf
    elif where == "beta_nan":
        beta[7] = np.nan
    else:
        beta[5] = 100.0  # exp(100) overflows fp32
    h = ctypes.c_void_p()
    st = lib.rw4_transform_givens(128, 1, pairs.ctypes.data, theta.ctypes.data, beta.ctypes.data, None,
                                  ctypes.byref(h))
    assert st == ARG
    assert not h.value


def test_table_transforms_bound_k():
    h = ctypes.c_void_p()
    big = 1 << 25
    assert lib.rw4_transform_hadamard_signed(big, 128, FAKE, None, ctypes.byref(h)) == SHAPE
    assert lib.rw4_transform_givens(big, 8, FAKE, FAKE, FAKE, None, ctypes.byref(h)) == SHAPE
    assert lib.rw4_transform_givens_f16(big, 8, FAKE, FAKE, FAKE, None, ctypes.byref(h)) == SHAPE
    assert not h.value


def test_binding_refuses_host_tensors():
    """A host tensor's address must never reach a kernel: every compute call
    of the binding refuses non-GPU tensors before calling the library."""
    torch = pytest.importorskip("torch")
    t = rw4.Transform.hadamard(256, 128)
    x = torch.zeros((4, 256), dtype=torch.float32)
    q = torch.zeros((4, 128), dtype=torch.uint8)
    s = torch.zeros((4, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        rw4.quantize_act(t, x)
    with pytest.raises(ValueError, match="GPU"):
        rw4.pack_weight(t, x.t())
    with pytest.raises(ValueError, match="GPU"):
        rw4.dequantize(q, s, torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        rw4.w4a4_gemm(q, s, q, s, torch.float32)
    t.close()


def test_rotate_act_validation():
    """rotate_act rejects what quantize_act rejects, before any device work."""
    f = lib.rw4_rotate_act
    assert f(None, FAKE, 1, 4, 256, FAKE, 1, 256, None) == ARG          # no transform
    st, h = _had(256, 128)
    assert st == OK
    try:
        assert f(h, FAKE, 7, 4, 256, FAKE, 1, 256, None) == ARG         # unknown input dtype
        assert f(h, FAKE, 1, 4, 256, FAKE, 9, 256, None) == ARG         # unknown output dtype
        assert f(h, FAKE, 1, -1, 256, FAKE, 1, 256, None) == SHAPE      # negative M
        assert f(h, None, 1, 0, 256, None, 1, 256, None) == OK          # empty: nothing to do
        assert f(h, None, 1, 4, 256, FAKE, 1, 256, None) == ARG         # null input
        assert f(h, FAKE, 1, 4, 200, FAKE, 1, 256, None) == ARG         # ldx < K
        assert f(h, FAKE, 1, 4, 256, FAKE, 1, 100, None) == ARG         # ldo < K
        assert f(h, FAKE + 2, 1, 4, 256, FAKE, 1, 256, None) == ARG     # misaligned input
        assert f(h, FAKE, 1, 4, 260, FAKE, 1, 256, None) == ARG         # row pitch not 16-byte aligned
    finally:
        lib.rw4_transform_destroy(h)


def test_every_entry_point_declares_its_argument_types():
    """Every C call taking pointers has ctypes argument types: without them
    ctypes passes Python ints as 32-bit C ints and device pointers get truncated."""
    for n in rw4.EXPORTED_SYMBOLS:
        if n in ("rw4_version",):
            continue
        assert getattr(lib, n).argtypes is not None, n


def test_reorder_entry_points_validation():
    assert lib.rw4_rrs_reorder_workspace_bytes(100) == 0
    assert lib.rw4_rrs_reorder_workspace_bytes(4096) == (256 + 1) * 4096 * 4 + 32 * 4
    f = lib.rw4_quantize_act_rrs_reorder
    assert f(None, FAKE, 1, 4, 4096, FAKE, FAKE, FAKE, FAKE, None) == ARG
    st, h = _had(8192, 8192)
    assert st == OK
    try:  # K = 8192 is beyond the reorder kernels
        assert f(h, FAKE, 1, 4, 8192, FAKE, FAKE, FAKE, FAKE, None) == UNSUP
    finally:
        lib.rw4_transform_destroy(h)
    st, h = _had(4096, 4096)
    try:
        assert f(h, FAKE, 1, 0, 4096, None, None, None, None, None) == OK      # empty
        assert f(h, FAKE, 1, 4, 4096, FAKE, FAKE, FAKE, None, None) == ARG     # no workspace
        assert f(h, FAKE, 1, 4, 4096, FAKE, FAKE, None, FAKE, None) == ARG     # no order
        assert f(h, FAKE, 1, -1, 4096, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
        assert lib.rw4_pack_weight_per_channel(h, FAKE, 1, 4, 0, 1, FAKE, FAKE, None) == ARG  # stride 0
    finally:
        lib.rw4_transform_destroy(h)
    p = lib.rw4_permute_codes
    assert p(FAKE, 4, 100, FAKE, FAKE + 64, None) == SHAPE
    assert p(FAKE, 4, 16384, FAKE, FAKE + 64, None) == SHAPE
    assert p(FAKE, 0, 128, None, None, None) == OK
    assert p(FAKE, 4, 128, FAKE, FAKE, None) == ARG   # in place
    assert p(FAKE, 4, 128, None, FAKE + 64, None) == ARG


def test_decode_fused_validation():
    """decode_fused: at most 16 rows, block-128 Hadamard or Givens, the
    checks of quantize_act and w4a4_gemm, all before any device work."""
    f = lib.rw4_decode_fused
    assert f(None, FAKE, 1, 4, 256, FAKE, FAKE, 64, FAKE, 1, 64, None) == ARG       # no transform
    st, h = _had(256, 128)
    assert st == OK
    try:
        assert f(h, FAKE, 7, 4, 256, FAKE, FAKE, 64, FAKE, 1, 64, None) == ARG      # unknown x dtype
        assert f(h, FAKE, 1, 4, 256, FAKE, FAKE, 64, FAKE, 9, 64, None) == ARG      # unknown y dtype
        assert f(h, FAKE, 1, 17, 256, FAKE, FAKE, 64, FAKE, 1, 64, None) == SHAPE   # more than 16 rows
        assert f(h, FAKE, 1, -1, 256, FAKE, FAKE, 64, FAKE, 1, 64, None) == SHAPE
        assert f(h, FAKE, 1, 4, 256, FAKE, FAKE, -1, FAKE, 1, 64, None) == SHAPE
        assert f(h, None, 1, 0, 256, None, None, 64, None, 1, 64, None) == OK       # empty
        assert f(h, None, 1, 4, 256, None, None, 0, None, 1, 0, None) == OK         # no outputs
        assert f(h, None, 1, 4, 256, FAKE, FAKE, 64, FAKE, 1, 64, None) == ARG      # null x
        assert f(h, FAKE, 1, 4, 256, FAKE, None, 64, FAKE, 1, 64, None) == ARG      # null scales
        assert f(h, FAKE, 1, 4, 200, FAKE, FAKE, 64, FAKE, 1, 64, None) == ARG      # ldx < K
        assert f(h, FAKE, 1, 4, 256, FAKE, FAKE, 64, FAKE, 1, 32, None) == ARG      # ldy < N
        assert f(h, FAKE, 1, 4, 260, FAKE, FAKE, 64, FAKE, 1, 64, None) == ARG      # row pitch not 16-byte aligned
        assert f(h, FAKE, 1, 4, 256, FAKE + 4, FAKE, 64, FAKE, 1, 64, None) == ARG  # misaligned weights
    finally:
        lib.rw4_transform_destroy(h)
    st, h = _had(512, 256)
    assert st == OK
    try:
        assert f(h, FAKE, 1, 4, 512, FAKE, FAKE, 64, FAKE, 1, 64, None) == UNSUP    # block 256
    finally:
        lib.rw4_transform_destroy(h)


def test_asym_entry_points_validation():
    """The asymmetric calls: block-128 Hadamard only, groups of 128, null and alignment checks."""
    f = lib.rw4_quantize_act_asym
    assert f(None, FAKE, 1, 4, 256, FAKE, FAKE, FAKE, None) == ARG          # no transform
    st, h = _had(256, 128)
    assert st == OK
    try:
        assert f(h, FAKE, 7, 4, 256, FAKE, FAKE, FAKE, None) == ARG         # unknown dtype
        assert f(h, FAKE, 1, -1, 256, FAKE, FAKE, FAKE, None) == SHAPE
        assert f(h, None, 1, 0, 256, None, None, None, None) == OK          # empty
        assert f(h, FAKE, 1, 4, 256, FAKE, FAKE, None, None) == ARG         # no zero points
        assert f(h, FAKE, 1, 4, 200, FAKE, FAKE, FAKE, None) == ARG         # ldx < K
        assert f(h, FAKE, 1, 4, 256, FAKE, FAKE, FAKE + 4, None) == ARG     # misaligned za
    finally:
        lib.rw4_transform_destroy(h)
    st, h = _had(512, 512)
    assert st == OK
    try:
        assert f(h, FAKE, 1, 4, 512, FAKE, FAKE, FAKE, None) == UNSUP       # block 512
    finally:
        lib.rw4_transform_destroy(h)
    c = lib.rw4_weight_code_sums
    assert c(FAKE, 4, 100, FAKE, None) == SHAPE
    assert c(FAKE, 0, 128, None, None) == OK
    assert c(None, 4, 128, FAKE, None) == ARG
    g = lib.rw4_w4a4_gemm_asym
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 200, FAKE, 1, 4, None) == SHAPE    # K % 128
    assert g(FAKE, FAKE, None, FAKE, FAKE, FAKE, 4, 4, 256, FAKE, 1, 4, None) == ARG     # no za
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 4, 256, FAKE, 1, 4, None) == ARG     # no cw
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 256, FAKE, 9, 4, None) == ARG     # bad dtype
    assert g(None, None, None, None, None, None, 0, 4, 256, None, 1, 4, None) == OK      # empty
    d = lib.rw4_dequantize_asym
    assert d(FAKE, FAKE, FAKE, 4, 200, FAKE, 1, 256, None) == SHAPE
    assert d(FAKE, FAKE, None, 4, 256, FAKE, 1, 256, None) == ARG
    assert d(FAKE, FAKE, FAKE, 4, 256, FAKE, 1, 100, None) == ARG                        # ldo < K


def test_mixed_entry_points_validation():
    """8-bit groups: block-128 Hadamard only, n8 <= K/128, null checks before device work."""
    f = lib.rw4_quantize_act_mixed
    assert f(None, FAKE, 1, 4, 256, FAKE, 1, FAKE, FAKE, None) == ARG
    st, h = _had(256, 128)
    assert st == OK
    try:
        assert f(h, FAKE, 1, 4, 256, FAKE, 3, FAKE, FAKE, None) == SHAPE     # n8 > K / 128
        assert f(h, FAKE, 1, 4, 256, FAKE, -1, FAKE, FAKE, None) == SHAPE
        assert f(h, FAKE, 1, 4, 256, None, 1, FAKE, FAKE, None) == ARG       # no slot map
        assert f(h, None, 1, 0, 256, None, 1, None, None, None) == OK        # empty
        assert f(h, FAKE, 1, 4, 200, FAKE, 1, FAKE, FAKE, None) == ARG       # ldx < K
    finally:
        lib.rw4_transform_destroy(h)
    st, h = _had(512, 256)
    try:
        assert f(h, FAKE, 1, 4, 512, FAKE, 1, FAKE, FAKE, None) == UNSUP
    finally:
        lib.rw4_transform_destroy(h)
    e = lib.rw4_extend_weight_groups
    assert e(FAKE, FAKE, 4, 100, FAKE, 1, FAKE, FAKE, None) == SHAPE
    assert e(FAKE, FAKE, 4, 256, FAKE, 3, FAKE, FAKE, None) == SHAPE
    assert e(FAKE, FAKE, 4, 256, None, 1, FAKE, FAKE, None) == ARG
    assert e(FAKE, FAKE, 0, 256, None, 1, None, None, None) == OK
