"""Rotated W4A4 hot path on AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over ``librw4.so`` (C ABI in ``include/rw4.h``): it
takes torch tensors, passes their device pointers, sizes and the current
HIP stream, allocates the outputs with torch and turns a non-OK status into
``RuntimeError``.  Every step of the path runs in the library's HIP
kernels; there is no fallback.  Importing fails loudly when the library has
not been built (``python -m rotated_w4a4_amd._build``).

    t = Transform.hadamard(K, block=128)             # or .hadamard(K, 128, signs), Transform.givens(...)
    qw, sw = pack_weight(t, w)                       # w: [K, N] (offline)
    qa, sa = quantize_act(t, x)                      # x: [M, K] bf16 / fp32
    y = w4a4_gemm(qa, sa, qw, sw, torch.bfloat16)    # [M, N]

    step = prepare_w4a4_gemm(qa, sa, qw, sw, out=y)  # checked once; step() launches again
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "LIB_PATH", "lib", "RW4Error", "Transform", "quantize_act", "pack_weight", "w4a4_gemm",
    "dequantize", "rotate_act", "Call", "prepare_quantize_act", "prepare_w4a4_gemm", "prepare_dequantize",
    "prepare_rotate_act", "quantize_act_static", "quantize_act_rrs_reorder", "pack_weight_per_channel",
    "permute_codes", "prepare_permute_codes", "decode_fused", "prepare_decode_fused",
    "quantize_act_asym", "prepare_quantize_act_asym", "weight_code_sums", "w4a4_gemm_asym", "prepare_w4a4_gemm_asym",
    "dequantize_asym", "mixed_tables", "quantize_act_mixed", "prepare_quantize_act_mixed", "extend_weight_groups",
    "status_str", "version", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librw4.so")

RW4_OK = 0
RW4_F32, RW4_BF16 = 0, 1
MODES = {"group128": 0, "rrs": 1}

EXPORTED_SYMBOLS = (
    "rw4_transform_hadamard", "rw4_transform_hadamard_signed", "rw4_transform_givens",
    "rw4_transform_givens_f16",
    "rw4_transform_destroy", "rw4_transform_k", "rw4_quantize_act", "rw4_pack_weight",
    "rw4_dequantize", "rw4_w4a4_gemm", "rw4_quantize_act_g", "rw4_pack_weight_g",
    "rw4_dequantize_g", "rw4_w4a4_gemm_g", "rw4_rotate_act", "rw4_quantize_act_static", "rw4_status_str",
    "rw4_version", "rw4_rrs_reorder_workspace_bytes", "rw4_quantize_act_rrs_reorder", "rw4_pack_weight_per_channel",
    "rw4_permute_codes", "rw4_decode_fused", "rw4_quantize_act_asym", "rw4_weight_code_sums", "rw4_w4a4_gemm_asym",
    "rw4_dequantize_asym", "rw4_quantize_act_mixed", "rw4_extend_weight_groups",
)


def _load():
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7)
    # as the system ROCm that librw4.so links against.  Loading torch first
    # makes the process use one runtime, torch's, for both; the other order
    # leaves torch on a runtime it was not built for.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m rotated_w4a4_amd._build` "
            "(the HIP library is required; there is no CPU fallback)")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
lib.rw4_status_str.restype = ctypes.c_char_p
lib.rw4_status_str.argtypes = [ctypes.c_int]
lib.rw4_version.restype = ctypes.c_char_p
lib.rw4_transform_hadamard.argtypes = [_i64, _i32, _p, ctypes.POINTER(_p)]
lib.rw4_transform_hadamard_signed.argtypes = [_i64, _i32, _p, _p, ctypes.POINTER(_p)]
lib.rw4_transform_givens.argtypes = [_i64, _i32, _p, _p, _p, _p, ctypes.POINTER(_p)]
lib.rw4_transform_givens_f16.argtypes = [_i64, _i32, _p, _p, _p, _p, ctypes.POINTER(_p)]
lib.rw4_transform_destroy.argtypes = [_p]
lib.rw4_transform_k.argtypes = [_p]
lib.rw4_transform_k.restype = _i64
lib.rw4_quantize_act.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _p, _p, _p, _p]
lib.rw4_pack_weight.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _p]
lib.rw4_w4a4_gemm.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, ctypes.c_int, _i64, _p]
lib.rw4_dequantize.argtypes = [_p, _p, _i64, _i64, _p, ctypes.c_int, _i64, _p]
lib.rw4_quantize_act_g.argtypes = [_p, ctypes.c_int, _i32, _p, ctypes.c_int, _i64, _i64, _p, _p, _p, _p]
lib.rw4_pack_weight_g.argtypes = [_p, _i32, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _p]
lib.rw4_w4a4_gemm_g.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i32, _p, ctypes.c_int, _i64, _p]
lib.rw4_dequantize_g.argtypes = [_p, _p, _i64, _i64, _i32, _p, ctypes.c_int, _i64, _p]
lib.rw4_rotate_act.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _p, ctypes.c_int, _i64, _p]
lib.rw4_quantize_act_static.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _p, _p, _p]
lib.rw4_rrs_reorder_workspace_bytes.argtypes = [_i64]
lib.rw4_rrs_reorder_workspace_bytes.restype = _i64
lib.rw4_quantize_act_rrs_reorder.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _p, _p, _p, _p, _p]
lib.rw4_pack_weight_per_channel.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _i64, _p, _p, _p]
lib.rw4_permute_codes.argtypes = [_p, _i64, _i64, _p, _p, _p]
lib.rw4_decode_fused.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _p, _p, _i64, _p, ctypes.c_int, _i64, _p]
lib.rw4_quantize_act_asym.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _p, _p, _p, _p]
lib.rw4_weight_code_sums.argtypes = [_p, _i64, _i64, _p, _p]
lib.rw4_w4a4_gemm_asym.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, ctypes.c_int, _i64, _p]
lib.rw4_dequantize_asym.argtypes = [_p, _p, _p, _i64, _i64, _p, ctypes.c_int, _i64, _p]
lib.rw4_quantize_act_mixed.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _p, _i64, _p, _p, _p]
lib.rw4_extend_weight_groups.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p]
for _name in EXPORTED_SYMBOLS:
    if _name not in ("rw4_status_str", "rw4_version", "rw4_transform_k", "rw4_rrs_reorder_workspace_bytes"):
        getattr(lib, _name).restype = ctypes.c_int


class RW4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)}")
        self.status = status


def status_str(status: int) -> str:
    return lib.rw4_status_str(int(status)).decode()


def version() -> str:
    return lib.rw4_version().decode()


def _check(status: int, what: str):
    if status != RW4_OK:
        raise RW4Error(status, what)


def _torch():
    import torch
    return torch


_raw_stream = None


def _stream(dev: int) -> int:
    """The current HIP stream of device index `dev`, as the raw handle the C ABI takes."""
    global _raw_stream
    if _raw_stream is None:
        torch = _torch()
        fast = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = fast if fast is not None else (lambda d: torch.cuda.current_stream(d).cuda_stream)
    return _raw_stream(dev)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RW4_F32
    if t.dtype == torch.bfloat16:
        return RW4_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _on_gpu(name, t, dev=None) -> int:
    """A tensor the kernels will touch: on a GPU (device index `dev` if given); returns its index."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    d = t.get_device()
    if dev is not None and d != dev:
        raise ValueError(f"{name} is on cuda:{d}, expected cuda:{dev}")
    return d


def _out(name, t, shape, dtype, dev):
    """A caller-provided output: exact shape and dtype, contiguous, on GPU `dev`."""
    _on_gpu(name, t, dev)
    if t.shape != shape or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


class Call:
    """One library call with its arguments checked and marshalled once.

    Calling it launches the kernels again on the current stream of the
    tensors' GPU, with the same buffers (a serving loop reuses its buffers
    every step; this skips the per-call checks, which cost the host more
    time than a decode-sized kernel runs).  It holds references to every
    tensor and transform it uses, so they stay allocated while it exists.
    """

    __slots__ = ("_fn", "_args", "_dev", "_what", "_keep", "result")

    def __init__(self, fn, args, dev, what, keep, result):
        self._fn, self._args, self._dev, self._what = fn, args, dev, what
        self._keep, self.result = keep, result

    def __call__(self):
        status = self._fn(*self._args, _stream(self._dev))
        if status != RW4_OK:
            raise RW4Error(status, self._what)
        return self.result


class Transform:
    """Owns a library transform object (a host struct plus device tables)."""

    def __init__(self, handle: ctypes.c_void_p, K: int, kind: str):
        self._h = handle
        self.K = K
        self.kind = kind

    @property
    def handle(self):
        return self._h

    @classmethod
    def hadamard(cls, K: int, block: int = 128, signs=None, stream=None) -> "Transform":
        """Block Hadamard; with ``signs`` (K values of +1/-1) the randomized form."""
        h = ctypes.c_void_p()
        if signs is None:
            _check(lib.rw4_transform_hadamard(int(K), int(block), stream, ctypes.byref(h)),
                   "rw4_transform_hadamard")
            return cls(h, int(K), f"hadamard{block}")
        signs = np.ascontiguousarray(signs, dtype=np.int8)
        if signs.shape != (int(K),):
            raise ValueError("signs must have K entries")
        _check(lib.rw4_transform_hadamard_signed(int(K), int(block), signs.ctypes.data, stream,
                                                 ctypes.byref(h)),
               "rw4_transform_hadamard_signed")
        return cls(h, int(K), f"hadamard{block}_signed")

    @classmethod
    def givens(cls, K: int, pairs, theta, beta, stream=None) -> "Transform":
        """pairs uint8 [K/128, L, 64, 2] (0xFF = empty), theta [K/128, L, 64], beta fp32 [K].

        theta as float16 uses the half-precision angle entry point; anything
        else is converted to float32."""
        pairs = np.ascontiguousarray(pairs, dtype=np.uint8)
        half = np.asarray(theta).dtype == np.float16
        theta = np.ascontiguousarray(theta, dtype=np.float16 if half else np.float32)
        beta = np.ascontiguousarray(beta, dtype=np.float32)
        G = int(K) // 128
        L = pairs.shape[1]
        if pairs.shape != (G, L, 64, 2) or theta.shape != (G, L, 64) or beta.shape != (int(K),):
            raise ValueError("pairs/theta/beta shapes do not match K")
        h = ctypes.c_void_p()
        fn = lib.rw4_transform_givens_f16 if half else lib.rw4_transform_givens
        _check(fn(int(K), int(L), pairs.ctypes.data, theta.ctypes.data, beta.ctypes.data, stream,
                  ctypes.byref(h)),
               "rw4_transform_givens")
        return cls(h, int(K), f"givens{L}" + ("_f16" if half else ""))

    def close(self):
        if self._h is not None and self._h.value:
            _check(lib.rw4_transform_destroy(self._h), "rw4_transform_destroy")
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def quantize_act(t: Transform, x, mode: str = "group128", qa=None, sa=None, workspace=None,
                 group: int = 128):
    """Transform + INT4-quantize activations x [M, K] (bf16/fp32, unit stride in K).

    Returns (qa uint8 [M, K/2], sa fp32 [M, K/group]).  For mode="rrs" a
    workspace of K/128 fp32 is allocated unless given (it receives s_g).
    mode "group128" means per-group scales, of `group` channels.
    """
    return prepare_quantize_act(t, x, mode, qa, sa, workspace, group)()


def prepare_quantize_act(t: Transform, x, mode: str = "group128", qa=None, sa=None, workspace=None,
                         group: int = 128) -> Call:
    """quantize_act checked and marshalled once; calling the result runs it (returns (qa, sa))."""
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    dev = _on_gpu("x", x)
    M, K = x.shape
    if K != t.K:
        raise ValueError(f"x has {K} channels, the transform {t.K}")
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}")
    if group not in (64, 128, 256) or K % group:
        raise ValueError("group must be 64, 128 or 256 and divide K")
    G = K // 128
    if qa is None:
        qa = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty((M, K // group), dtype=torch.float32, device=x.device)
    _out("qa", qa, (M, K // 2), torch.uint8, dev)
    _out("sa", sa, (M, K // group), torch.float32, dev)
    if mode == "rrs":
        if workspace is None:
            workspace = torch.empty((max(G, 4),), dtype=torch.float32, device=x.device)
        _on_gpu("workspace", workspace, dev)
        if workspace.dtype != torch.float32 or not workspace.is_contiguous() or workspace.numel() < G:
            raise ValueError(f"workspace must be a contiguous float32 tensor of at least {G} elements")
    args = (t.handle, MODES[mode], group, x.data_ptr(), _dtype_code(x), M, x.stride(0), qa.data_ptr(),
            sa.data_ptr(), workspace.data_ptr() if workspace is not None else None)
    return Call(lib.rw4_quantize_act_g, args, dev, "rw4_quantize_act", (t, x, workspace), (qa, sa))


def quantize_act_static(t: Transform, x, mode: str = "group128", qa=None, sa=None):
    """quantize_act through the allocation-free entry point: no workspace; in
    "rrs" mode the group maxima use the library's static per-GPU scratch
    (K <= 8192).  Calls overlapping on one GPU race (shared scratch)."""
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    dev = _on_gpu("x", x)
    M, K = x.shape
    if K != t.K:
        raise ValueError(f"x has {K} channels, the transform {t.K}")
    if mode not in MODES:
        raise ValueError(f"mode must be one of {sorted(MODES)}")
    if qa is None:
        qa = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    _out("qa", qa, (M, K // 2), torch.uint8, dev)
    _out("sa", sa, (M, K // 128), torch.float32, dev)
    _check(lib.rw4_quantize_act_static(t.handle, MODES[mode], x.data_ptr(), _dtype_code(x), M, x.stride(0),
                                       qa.data_ptr(), sa.data_ptr(), _stream(dev)),
           "rw4_quantize_act_static")
    return qa, sa


def quantize_act_rrs_reorder(t: Transform, x, qa=None, sa=None, order=None, workspace=None):
    """Rotated Runtime Smooth with the channel reorder: returns (qa, sa, order).

    qa holds the codes in the reordered channel order; order (int32 [K]) is
    the permutation to apply to the weights' codes (permute_codes)."""
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    dev = _on_gpu("x", x)
    M, K = x.shape
    if K != t.K:
        raise ValueError(f"x has {K} channels, the transform {t.K}")
    if qa is None:
        qa = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    if order is None:
        order = torch.empty((K,), dtype=torch.int32, device=x.device)
    nbytes = int(lib.rw4_rrs_reorder_workspace_bytes(K))
    if workspace is None:
        workspace = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=x.device)
    _out("qa", qa, (M, K // 2), torch.uint8, dev)
    _out("sa", sa, (M, K // 128), torch.float32, dev)
    _out("order", order, (K,), torch.int32, dev)
    _on_gpu("workspace", workspace, dev)
    if not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a contiguous tensor of at least {nbytes} bytes")
    _check(lib.rw4_quantize_act_rrs_reorder(t.handle, x.data_ptr(), _dtype_code(x), M, x.stride(0), qa.data_ptr(),
                                            sa.data_ptr(), order.data_ptr(), workspace.data_ptr(), _stream(dev)),
           "rw4_quantize_act_rrs_reorder")
    return qa, sa, order


def pack_weight_per_channel(t: Transform, w, layout: str = "kn", qw=None, sw=None):
    """pack_weight with one scale per output channel (stored in every group column)."""
    torch = _torch()
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    dev = _on_gpu("w", w)
    if layout == "kn":
        K, N = w.shape
        sk, sn = w.stride(0), w.stride(1)
    elif layout == "nk":
        N, K = w.shape
        sn, sk = w.stride(0), w.stride(1)
    else:
        raise ValueError(layout)
    if K != t.K:
        raise ValueError(f"w has {K} input channels, the transform {t.K}")
    if qw is None:
        qw = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    if sw is None:
        sw = torch.empty((N, K // 128), dtype=torch.float32, device=w.device)
    _out("qw", qw, (N, K // 2), torch.uint8, dev)
    _out("sw", sw, (N, K // 128), torch.float32, dev)
    _check(lib.rw4_pack_weight_per_channel(t.handle, w.data_ptr(), _dtype_code(w), N, sk, sn, qw.data_ptr(),
                                           sw.data_ptr(), _stream(dev)),
           "rw4_pack_weight_per_channel")
    return qw, sw


def permute_codes(q, order, out=None):
    """out[r, j] = code order[j] of row r of the packed codes q [rows, K/2]."""
    return prepare_permute_codes(q, order, out)()


def prepare_permute_codes(q, order, out=None) -> Call:
    torch = _torch()
    rows, Kh = q.shape
    K = 2 * Kh
    dev = _on_gpu("q", q)
    _on_gpu("order", order, dev)
    if q.dtype != torch.uint8 or not q.is_contiguous():
        raise ValueError("q must be a contiguous uint8 tensor")
    if order.shape != (K,) or order.dtype != torch.int32 or not order.is_contiguous():
        raise ValueError(f"order must be a contiguous int32 tensor of {K} entries")
    if out is None:
        out = torch.empty_like(q)
    _out("out", out, (rows, Kh), torch.uint8, dev)
    args = (q.data_ptr(), rows, K, order.data_ptr(), out.data_ptr())
    return Call(lib.rw4_permute_codes, args, dev, "rw4_permute_codes", (q, order), out)


def decode_fused(t: Transform, x, qw, sw, out_dtype=None, out=None):
    """One decode step in one launch: y = w4a4_gemm(quantize_act(t, x), qw, sw), 1..16 rows."""
    return prepare_decode_fused(t, x, qw, sw, out_dtype, out)()


def prepare_decode_fused(t: Transform, x, qw, sw, out_dtype=None, out=None) -> Call:
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    dev = _on_gpu("x", x)
    M, K = x.shape
    if K != t.K:
        raise ValueError(f"x has {K} channels, the transform {t.K}")
    N = qw.shape[0]
    for name, tns, dt in (("qw", qw, torch.uint8), ("sw", sw, torch.float32)):
        _on_gpu(name, tns, dev)
        if tns.dtype != dt or not tns.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    if qw.shape != (N, K // 2) or sw.shape != (N, K // 128):
        raise ValueError("weight shapes do not match K (groups of 128)")
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _on_gpu("out", out, dev)
    if out.dim() != 2 or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be [{M}, {N}] with unit stride along N")
    args = (t.handle, x.data_ptr(), _dtype_code(x), M, x.stride(0), qw.data_ptr(), sw.data_ptr(), N,
            out.data_ptr(), _dtype_code(out), out.stride(0))
    return Call(lib.rw4_decode_fused, args, dev, "rw4_decode_fused", (t, x, qw, sw), out)


def pack_weight(t: Transform, w, layout: str = "kn", qw=None, sw=None, group: int = 128):
    """Transform + INT4-pack weights. layout "kn": w is [K, N]; "nk": w is [N, K] (nn.Linear).

    Returns (qw uint8 [N, K/2], sw fp32 [N, K/group]).
    """
    torch = _torch()
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    dev = _on_gpu("w", w)
    if layout == "kn":
        K, N = w.shape
        sk, sn = w.stride(0), w.stride(1)
    elif layout == "nk":
        N, K = w.shape
        sn, sk = w.stride(0), w.stride(1)
    else:
        raise ValueError(layout)
    if K != t.K:
        raise ValueError(f"w has {K} input channels, the transform {t.K}")
    if group not in (64, 128, 256) or K % group:
        raise ValueError("group must be 64, 128 or 256 and divide K")
    if qw is None:
        qw = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    if sw is None:
        sw = torch.empty((N, K // group), dtype=torch.float32, device=w.device)
    _out("qw", qw, (N, K // 2), torch.uint8, dev)
    _out("sw", sw, (N, K // group), torch.float32, dev)
    _check(lib.rw4_pack_weight_g(t.handle, group, w.data_ptr(), _dtype_code(w), N, sk, sn, qw.data_ptr(),
                                 sw.data_ptr(), _stream(dev)),
           "rw4_pack_weight")
    return qw, sw


def rotate_act(t: Transform, x, out_dtype=None, out=None):
    """The transform alone: x R (Hadamard) or x R D^-1 (Givens), unquantized.

    x [M, K] (bf16/fp32, unit stride in K); returns out [M, K] in out_dtype
    (default bf16), e.g. queries rotated like the keys of an INT4 KV cache."""
    return prepare_rotate_act(t, x, out_dtype, out)()


def prepare_rotate_act(t: Transform, x, out_dtype=None, out=None) -> Call:
    """rotate_act checked and marshalled once; calling the result runs it (returns out)."""
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    dev = _on_gpu("x", x)
    M, K = x.shape
    if K != t.K:
        raise ValueError(f"x has {K} channels, the transform {t.K}")
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=x.device)
    _on_gpu("out", out, dev)
    if out.dim() != 2 or out.shape != (M, K) or out.stride(1) != 1:
        raise ValueError(f"out must be [{M}, {K}] with unit stride along K")
    args = (t.handle, x.data_ptr(), _dtype_code(x), M, x.stride(0), out.data_ptr(), _dtype_code(out),
            out.stride(0))
    return Call(lib.rw4_rotate_act, args, dev, "rw4_rotate_act", (t, x), out)


def _group_of(K, cols):
    if cols <= 0 or K % cols or (K // cols) not in (64, 128, 256):
        raise ValueError("scale columns do not give a group of 64, 128 or 256 channels")
    return K // cols


def dequantize(q, s, out_dtype=None, out=None):
    """x_hat [M, K] = codes * group scale (transformed domain), fp32 or bf16.

    The group size is K divided by the number of scale columns."""
    return prepare_dequantize(q, s, out_dtype, out)()


def prepare_dequantize(q, s, out_dtype=None, out=None) -> Call:
    """dequantize checked and marshalled once; calling the result runs it (returns out)."""
    torch = _torch()
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    M, Kh = q.shape
    K = Kh * 2
    if s.dim() != 2 or s.shape[0] != M:
        raise ValueError("scale shape does not match the codes")
    group = _group_of(K, s.shape[1])
    dev = _on_gpu("q", q)
    _on_gpu("s", s, dev)
    if q.dtype != torch.uint8 or s.dtype != torch.float32:
        raise ValueError("q must be uint8 and s float32")
    if not (q.is_contiguous() and s.is_contiguous()):
        raise ValueError("q and s must be contiguous")
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=q.device)
    _on_gpu("out", out, dev)
    if out.dim() != 2 or out.shape != (M, K) or out.stride(1) != 1:
        raise ValueError(f"out must be [{M}, {K}] with unit stride along K")
    args = (q.data_ptr(), s.data_ptr(), M, K, group, out.data_ptr(), _dtype_code(out), out.stride(0))
    return Call(lib.rw4_dequantize_g, args, dev, "rw4_dequantize", (q, s), out)


def quantize_act_asym(t: Transform, x, qa=None, sa=None, za=None):
    """Transform + asymmetric (s, z) INT4 in groups of 128 (block-128 Hadamard).

    Returns (qa uint8 [M, K/2] unsigned codes (stored form of rw4.h), sa fp32 [M, K/128], za fp32 [M, K/128])."""
    return prepare_quantize_act_asym(t, x, qa, sa, za)()


def prepare_quantize_act_asym(t: Transform, x, qa=None, sa=None, za=None) -> Call:
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    dev = _on_gpu("x", x)
    M, K = x.shape
    if K != t.K:
        raise ValueError(f"x has {K} channels, the transform {t.K}")
    G = K // 128
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device) if qa is None else qa
    sa = torch.empty((M, G), dtype=torch.float32, device=x.device) if sa is None else sa
    za = torch.empty((M, G), dtype=torch.float32, device=x.device) if za is None else za
    _out("qa", qa, (M, K // 2), torch.uint8, dev)
    _out("sa", sa, (M, G), torch.float32, dev)
    _out("za", za, (M, G), torch.float32, dev)
    args = (t.handle, x.data_ptr(), _dtype_code(x), M, x.stride(0), qa.data_ptr(), sa.data_ptr(), za.data_ptr())
    return Call(lib.rw4_quantize_act_asym, args, dev, "rw4_quantize_act_asym", (t, x), (qa, sa, za))


def weight_code_sums(qw, cw=None):
    """cw fp32 [N, K/128]: the sum of every 128-group of codes of the packed weights qw."""
    torch = _torch()
    N, Kh = qw.shape
    K = Kh * 2
    dev = _on_gpu("qw", qw)
    if qw.dtype != torch.uint8 or not qw.is_contiguous():
        raise ValueError("qw must be a contiguous uint8 tensor")
    cw = torch.empty((N, K // 128), dtype=torch.float32, device=qw.device) if cw is None else cw
    _out("cw", cw, (N, K // 128), torch.float32, dev)
    return Call(lib.rw4_weight_code_sums, (qw.data_ptr(), N, K, cw.data_ptr()), dev, "rw4_weight_code_sums",
                (qw,), cw)()


def w4a4_gemm_asym(qa, sa, za, qw, sw, cw, out_dtype=None, out=None):
    """Y [M, N] from asymmetric activations (qa, sa, za) and weights (qw, sw) with their code sums cw."""
    return prepare_w4a4_gemm_asym(qa, sa, za, qw, sw, cw, out_dtype, out)()


def prepare_w4a4_gemm_asym(qa, sa, za, qw, sw, cw, out_dtype=None, out=None) -> Call:
    torch = _torch()
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    M, Kh = qa.shape
    N = qw.shape[0]
    K = Kh * 2
    G = K // 128
    if K % 128 or qw.shape[1] != Kh or sa.shape != (M, G) or za.shape != (M, G) or sw.shape != (N, G) \
            or cw.shape != (N, G):
        raise ValueError("operand shapes do not match (groups of 128)")
    dev = _on_gpu("qa", qa)
    u8, f32 = torch.uint8, torch.float32
    for name, tns, dt in (("qa", qa, u8), ("sa", sa, f32), ("za", za, f32), ("qw", qw, u8), ("sw", sw, f32),
                          ("cw", cw, f32)):
        _on_gpu(name, tns, dev)
        if tns.dtype != dt or not tns.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    _on_gpu("out", out, dev)
    if out.dim() != 2 or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be [{M}, {N}] with unit stride along N")
    args = (qa.data_ptr(), sa.data_ptr(), za.data_ptr(), qw.data_ptr(), sw.data_ptr(), cw.data_ptr(), M, N, K,
            out.data_ptr(), _dtype_code(out), out.stride(0))
    return Call(lib.rw4_w4a4_gemm_asym, args, dev, "rw4_w4a4_gemm_asym", (qa, sa, za, qw, sw, cw), out)


def dequantize_asym(q, s, z, out_dtype=None, out=None):
    """x_hat [M, K] = s * (q - z) from the asymmetric form (groups of 128), fp32 or bf16."""
    torch = _torch()
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    M, Kh = q.shape
    K = Kh * 2
    if K % 128 or s.shape != (M, K // 128) or z.shape != (M, K // 128):
        raise ValueError("scale / zero-point shapes do not match the codes")
    dev = _on_gpu("q", q)
    for name, tns, dt in (("q", q, torch.uint8), ("s", s, torch.float32), ("z", z, torch.float32)):
        _on_gpu(name, tns, dev)
        if tns.dtype != dt or not tns.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    out = torch.empty((M, K), dtype=out_dtype, device=q.device) if out is None else out
    _on_gpu("out", out, dev)
    if out.dim() != 2 or out.shape != (M, K) or out.stride(1) != 1:
        raise ValueError(f"out must be [{M}, {K}] with unit stride along K")
    args = (q.data_ptr(), s.data_ptr(), z.data_ptr(), M, K, out.data_ptr(), _dtype_code(out), out.stride(0))
    return Call(lib.rw4_dequantize_asym, args, dev, "rw4_dequantize_asym", (q, s, z), out)()


def mixed_tables(K: int, groups8, device):
    """The device tables of a set of 8-bit groups: (slot_of_group int32 [K/128],
    groups8 int32 [n8]) for quantize_act_mixed and extend_weight_groups."""
    torch = _torch()
    G = K // 128
    groups8 = [int(g) for g in groups8]
    if len(set(groups8)) != len(groups8) or any(g < 0 or g >= G for g in groups8):
        raise ValueError(f"groups8 must be distinct group indices in [0, {G})")
    slot = np.full(G, -1, dtype=np.int32)
    for j, g in enumerate(groups8):
        slot[g] = j
    return (torch.from_numpy(slot).to(device),
            torch.tensor(groups8 if groups8 else [0], dtype=torch.int32, device=device)[:len(groups8)])


def quantize_act_mixed(t: Transform, x, slot_of_group, n8: int, qa=None, sa=None):
    """Block-128 Hadamard activations with n8 groups at 8 bits (two INT4 planes):
    qa uint8 [M, (K + 128 n8)/2], sa fp32 [M, K/128 + n8]."""
    return prepare_quantize_act_mixed(t, x, slot_of_group, n8, qa, sa)()


def prepare_quantize_act_mixed(t: Transform, x, slot_of_group, n8: int, qa=None, sa=None) -> Call:
    torch = _torch()
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    dev = _on_gpu("x", x)
    M, K = x.shape
    if K != t.K:
        raise ValueError(f"x has {K} channels, the transform {t.K}")
    G = K // 128
    _on_gpu("slot_of_group", slot_of_group, dev)
    if slot_of_group.dtype != torch.int32 or slot_of_group.shape != (G,) or not slot_of_group.is_contiguous():
        raise ValueError(f"slot_of_group must be a contiguous int32 tensor of {G} entries")
    Kx = K + 128 * int(n8)
    qa = torch.empty((M, Kx // 2), dtype=torch.uint8, device=x.device) if qa is None else qa
    sa = torch.empty((M, Kx // 128), dtype=torch.float32, device=x.device) if sa is None else sa
    _out("qa", qa, (M, Kx // 2), torch.uint8, dev)
    _out("sa", sa, (M, Kx // 128), torch.float32, dev)
    args = (t.handle, x.data_ptr(), _dtype_code(x), M, x.stride(0), slot_of_group.data_ptr(), int(n8), qa.data_ptr(),
            sa.data_ptr())
    return Call(lib.rw4_quantize_act_mixed, args, dev, "rw4_quantize_act_mixed", (t, x, slot_of_group), (qa, sa))


def extend_weight_groups(qw, sw, groups8, qw_ext=None, sw_ext=None):
    """qw/sw with the groups of groups8 (device int32 [n8]) appended: [N, (K + 128 n8)/2], [N, K/128 + n8]."""
    torch = _torch()
    N, Kh = qw.shape
    K = Kh * 2
    n8 = int(groups8.numel())
    dev = _on_gpu("qw", qw)
    for name, tns, dt in (("qw", qw, torch.uint8), ("sw", sw, torch.float32), ("groups8", groups8, torch.int32)):
        _on_gpu(name, tns, dev)
        if tns.dtype != dt or not tns.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    if sw.shape != (N, K // 128):
        raise ValueError("sw must be [N, K/128]")
    Kx = K + 128 * n8
    qw_ext = torch.empty((N, Kx // 2), dtype=torch.uint8, device=qw.device) if qw_ext is None else qw_ext
    sw_ext = torch.empty((N, Kx // 128), dtype=torch.float32, device=qw.device) if sw_ext is None else sw_ext
    _out("qw_ext", qw_ext, (N, Kx // 2), torch.uint8, dev)
    _out("sw_ext", sw_ext, (N, Kx // 128), torch.float32, dev)
    args = (qw.data_ptr(), sw.data_ptr(), N, K, groups8.data_ptr() if n8 else None, n8, qw_ext.data_ptr(),
            sw_ext.data_ptr())
    return Call(lib.rw4_extend_weight_groups, args, dev, "rw4_extend_weight_groups", (qw, sw, groups8),
                (qw_ext, sw_ext))()


def w4a4_gemm(qa, sa, qw, sw, out_dtype=None, out=None):
    """Y [M, N] = sum over groups of sa * sw * exact integer group products (fp32 epilogue).

    The group size is K divided by the number of scale columns."""
    return prepare_w4a4_gemm(qa, sa, qw, sw, out_dtype, out)()


def prepare_w4a4_gemm(qa, sa, qw, sw, out_dtype=None, out=None) -> Call:
    """w4a4_gemm checked and marshalled once; calling the result runs it (returns out)."""
    torch = _torch()
    if out_dtype is None:
        out_dtype = torch.bfloat16 if out is None else out.dtype
    M, Kh = qa.shape
    N = qw.shape[0]
    K = Kh * 2
    if qw.shape[1] != Kh or sa.dim() != 2 or sa.shape[0] != M or sw.shape != (N, sa.shape[1]):
        raise ValueError("operand shapes do not match")
    group = _group_of(K, sa.shape[1])
    dev = _on_gpu("qa", qa)
    u8, f32 = torch.uint8, torch.float32
    for name, tns, dt in (("qa", qa, u8), ("sa", sa, f32), ("qw", qw, u8), ("sw", sw, f32)):
        _on_gpu(name, tns, dev)
        if tns.dtype != dt or not tns.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    _on_gpu("out", out, dev)
    if out.dim() != 2 or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError(f"out must be [{M}, {N}] with unit stride along N")
    args = (qa.data_ptr(), sa.data_ptr(), qw.data_ptr(), sw.data_ptr(), M, N, K, group, out.data_ptr(),
            _dtype_code(out), out.stride(0))
    return Call(lib.rw4_w4a4_gemm_g, args, dev, "rw4_w4a4_gemm", (qa, sa, qw, sw), out)
