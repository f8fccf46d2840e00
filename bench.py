#!/usr/bin/env python3
"""Benchmark of the rotated W4A4 hot path on one MI355X.

One step = one pass of the whole online path over one batch: quantize_act
(load bf16 activations, block Walsh-Hadamard, group-128 absmax, INT4 RNE,
pack) followed by w4a4_gemm (FP6 MFMA on the exact codes, per-128-group
rescale, fp32 epilogue, bf16 output).  Weights are transformed and packed once before timing, as in
deployment (the offline step).  Default workload: LLaMA-3-8B q_proj prefill,
X 2048x4096 bf16 with channel outliers and spikes, W 4096x4096.

Inputs are resident in HBM before the timed region.  Independent buffer sets
(X, qa, sa, Y and a copy of the packed weights) are rotated so that at least
512 MB is touched between two uses of a set: the 256 MB Infinity Cache
cannot serve them.

Before the timed region the GPU runs the W warm-up steps and then further
untimed steps until it has been under load for at least --settle-ms (200
ms by default): its clocks ramp up under sustained load (the down_proj GEMM
takes 425 us cold and ~250 us settled), and a serving loop runs settled.
The warm-up actually run is reported as "warmup_run".
Prints one JSON line (stdout).  Per-kernel times come from HIP events
(created without the system-scope fence, so recording them flushes no
caches) recorded on the stream the library launches on, around the kernels
of every fourth timed step (recording them on every step would slow the
timed throughput itself by ~7 % at q_proj); the GEMM is the
dominant kernel and its int8 MFMA roofline (5 POPS dense) is reported (the
GEMM issues FP6 MFMAs; the fraction of their 10.1 PFLOP/s peak is given too),
the quantize kernel's HBM roofline beside it.  Steps are issued through
calls prepared once per buffer set (arguments checked and marshalled once,
as a serving loop reuses its buffers; `--launch eager` checks on every
call).  Each kernel is also timed
alone, 20 launches queued behind a 1 GiB device copy so that the host is
ahead of the GPU: for decode-sized and KV-cache steps, which are shorter
than the host's Python calls, that is the kernel's own duration and the
roofline uses it (HBM-bound: the weights or the cache are streamed once).
The CPU oracle is timed on a bounded sample of the same workload as a
reported baseline (not a target).  "device" names the GPU (architecture, CU
count, memory, HIP and ROCm versions) and the shader clock rocm-smi reports
right after the timed region.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A4 layer TOPS + quantize GB/s (% roofline) at LLaMA-3-8B q_proj shapes"
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
PEAK_I8_TOPS = 5000.0        # MI355X dense int8 (and FP8) MFMA: the INT4 GEMM's roofline
PEAK_F6_TFLOPS = 10100.0     # MI355X dense FP6 MFMA: the units the GEMM's products run on
MALL_FLUSH_BYTES = 512 << 20
EVENT_EVERY = 4              # timed steps per step instrumented with per-kernel events
SETTLE_MS = 200.0            # default untimed sustained load before timing (see warm_up)


def warm_up(run, args, torch):
    """The W untimed warm-up steps, then more untimed steps until the warm-up
    has kept the GPU busy for at least --settle-ms of wall time.  The GPU's
    clocks ramp up under sustained load: measured on the box, the down_proj
    GEMM takes 425 us in its first batch of launches and ~250 us after about
    25 ms of load (and is slow again after 2 s idle); the q_proj step drops
    from ~68 us to ~48 us within ~20 ms.  A serving loop runs at the settled
    clocks, so the timed region starts there.  Returns the warm-up steps run
    and the warm-up wall time in ms."""
    t0 = time.perf_counter()
    n = 0
    for _ in range(args.warmup):
        run(n)
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(8):
            run(n)
            n += 1
        torch.cuda.synchronize()
    return {"steps": n, "ms": (time.perf_counter() - t0) * 1e3}



def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvent:
    """A timing event of the HIP runtime that torch itself uses, created with
    hipEventDisableSystemFence: recording it does not write back and invalidate
    the caches (torch's default events do), so timing events inside the timed
    region do not slow the kernels they bracket."""

    _lib = None

    @classmethod
    def _hip(cls):
        if cls._lib is None:
            import torch
            lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = self._hip().hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        """stream: the hipStream_t handle (torch's current_stream().cuda_stream)."""
        rc = self._hip().hipEventRecord(self.h, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end):
        self._hip().hipEventSynchronize(end.h)
        f = ctypes.c_float()
        rc = self._hip().hipEventElapsedTime(ctypes.byref(f), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def __del__(self):
        if self._lib is not None and self.h:
            self._lib.hipEventDestroy(self.h)


_COVER = {}


def gpu_bound_us(torch, stream, fn, reps=20):
    """Average duration of `reps` launches fn(0..reps-1) with the host ahead of the GPU.

    A device copy of 1 GiB is queued first; while the GPU runs it, the host
    queues every launch, so no launch waits for the host (the Python binding
    takes longer per call than a decode-sized kernel runs, which inflates
    events recorded around single launches).  Returns (us per launch, whether
    the host finished queueing before the copy ended)."""
    if "src" not in _COVER:
        _COVER["src"] = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        _COVER["dst"] = torch.empty_like(_COVER["src"])
    c0, e0, e1 = HipEvent(), HipEvent(), HipEvent()
    torch.cuda.synchronize()
    c0.record(stream)
    _COVER["dst"].copy_(_COVER["src"])
    e0.record(stream)
    h0 = time.perf_counter()
    for i in range(reps):
        fn(i)
    e1.record(stream)
    host_ms = (time.perf_counter() - h0) * 1e3
    torch.cuda.synchronize()
    return e0.elapsed_ms(e1) * 1e3 / reps, host_ms < c0.elapsed_ms(e0)


def capture_steps(torch, step, nsets):
    """One HIP graph per buffer set holding that set's step (the library only launches
    kernels on the current stream: nothing to allocate, clear or synchronise inside)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # eager warm-up off the capture stream
        for i in range(nsets):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(nsets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed sustained load before timing, at least (after the warm-up steps)")
    ap.add_argument("--workload", default="q_proj",
                    choices=["q_proj", "down_proj", "rrs", "decode1", "decode4", "decode16", "decode32", "decode64",
                             "decode128", "decode256", "tiny", "kv", "rrs_reorder", "fused1", "fused2", "fused4",
                             "fused8", "fused16", "q_proj_asym", "down_proj_asym", "decode16_asym", "q_proj_mixed",
                             "down_proj_mixed"])
    ap.add_argument("--group", type=int, default=128, choices=[64, 128, 256],
                    help="quantization group size (block-128 Hadamard workloads for 64 and 256)")
    ap.add_argument("--launch", default="prepared", choices=["prepared", "eager", "graph"],
                    help="how a step is issued: calls prepared once per buffer set (arguments checked "
                         "and marshalled once, as a serving loop reuses its buffers), the checking Python "
                         "functions on every call, or one HIP graph replay per step (a replay costs more "
                         "GPU time than the two kernels of a decode step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows of the oracle sample (0 = auto)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


KERNEL_SOURCES = {
    "gemm_f8_kernel": ["gemm.hip", "rw4_device.h"],
    "gemm_f8p_kernel": ["gemm.hip", "rw4_device.h"],
    "gemm_small_kernel": ["gemm.hip", "rw4_device.h"],
    "decode_fused_kernel": ["gemm.hip", "rw4_device.h"],
    "quant_h128_act_kernel": ["quant.hip", "rw4_device.h"],
    "quant_h128_kernel": ["quant.hip", "rw4_device.h"],
    "quant_rrs_full_kernel": ["quant.hip", "rw4_device.h"],
    "quant_rowh_kernel": ["quant.hip", "rw4_device.h"],
    "quant_givens_kernel": ["quant.hip", "rw4_device.h"],
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "rotated_w4a4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if still valid.

    profiles/traffic.json holds, per (kernel, workload), the FETCH_SIZE and
    WRITE_SIZE counters (KiB per dispatch) already scaled by the copy
    calibration, and the hash of the kernel's sources when they were taken;
    a changed kernel gives None.
    """
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = table.get(f"{kernel}:{workload}")
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def workload(name):
    import datagen
    if name.startswith("decode"):
        return datagen.make("decode", M=int(name[len("decode"):]))
    return datagen.make(name)


def givens_table_bytes(K, layers):
    """The Givens lookup table the activation kernel reads: per (group, layer, slot) a
    2-byte pair index and an 8-byte (cos, sin), plus alpha^-1 per channel (4 bytes)."""
    return (K // 128) * layers * 64 * (2 + 8) + 4 * K


def algorithmic_bytes(wl, group=128):
    """Quantize: read X once (and the Givens table), write qa and sa.  GEMM: read qa, sa,
    qw, sw once, write Y."""
    M, K, N = wl.M, wl.K, wl.N
    G = K // group
    xb = 2 if wl.x_dtype == "bf16" else 4
    yb = 2 if wl.y_dtype == "bf16" else 4
    quant = M * K * xb + M * K // 2 + M * G * 4
    if wl.transform[0] == "givens":
        quant += givens_table_bytes(K, int(wl.transform[1]))
    gemm = M * K // 2 + M * G * 4 + N * K // 2 + N * G * 4 + M * N * yb
    return quant, gemm


def gemm_kernel_for(M, N, group=128):
    """The GEMM kernel the library runs for an M x N product: the small-M kernel up to 64
    rows, and up to 1024 rows (in 64-row chunks) while the 128 x 128-tile grid would have
    fewer than 128 blocks; the tiled kernel otherwise (its pipelined form for 128-wide groups)."""
    small = M <= 64 or (M <= 1024 and ((M + 127) // 128) * ((N + 127) // 128) < 128)
    if small:
        return "gemm_small_kernel"
    return "gemm_f8p_kernel" if group == 128 else "gemm_f8_kernel"


def cpu_baseline(wl, rows):
    """The oracle as it stands on a sample of `rows` tokens: quantize_act + w4a4_gemm.

    Weights are packed by the oracle beforehand (offline, not timed), as on
    the GPU.  For Rotated Runtime Smooth the group maxima need every token,
    so the sample's maxima are taken over the sample.
    """
    import oracle
    from tests.helpers import spec_of
    spec = spec_of(wl)
    w = oracle.pack_weight(wl.w, spec)
    x = wl.x[:rows]
    t0 = time.perf_counter()
    a = oracle.quantize_act(x, spec, wl.mode)
    oracle.w4a4_gemm(a["qa"], a["sa"], w["qw"], w["sw"], wl.y_dtype)
    dt = time.perf_counter() - t0
    return dt, blas_info()["threads"]


def blas_info():
    """The BLAS numpy runs the oracle's products on, and its thread count."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            b = blas[0]
            return {"threads": int(b.get("num_threads", 1)),
                    "library": f"{b.get('internal_api', '?')} {b.get('version', '')}".strip(),
                    "file": os.path.basename(b.get("filepath", ""))}
    except Exception:
        pass
    return {"threads": len(os.sched_getaffinity(0)), "library": "unknown", "file": ""}


def device_info(torch):
    """The GPU the line was measured on: name, architecture, CU count, memory,
    the HIP runtime torch was built against, and the shader clock that
    rocm-smi reports right after the timed region (None when unavailable)."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": torch.cuda.get_device_name(0), "arch": getattr(p, "gcnArchName", None),
            "cus": p.multi_processor_count, "memory_gib": round(p.total_memory / 2**30, 1),
            "hip": torch.version.hip, "rocm": None, "sclk_mhz": None}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        cards = json.loads(r.stdout) if r.returncode == 0 else {}
        for card in cards.values():
            for k, v in card.items():
                if "sclk" in k.lower() and "speed" in k.lower():
                    info["sclk_mhz"] = float(str(v).strip("()Mhz").split()[0])
                    break
            break
    except Exception:
        pass
    return info


def emit(out, torch):
    """print the result line, with the device it was measured on"""
    if "device" not in out:
        out["device"] = device_info(torch)
    print(json.dumps(out), flush=True)


def spread(xs):
    """median, p10 and p90 of a list of per-launch durations (us)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


KV_METRIC = "INT4 KV-cache quantize + dequantize GB/s (block-128 Hadamard per head) at 4096 tokens x 8 heads x 128"


def main_kv(args, torch, rw4, gu, dev):
    """The INT4 KV-cache use: quantize_act writes the cache, dequantize reads
    it back (bf16).  One step = both calls over 4096 tokens x 1024 channels."""
    import datagen
    wl = datagen.make("kv")
    M, K, grp = wl.M, wl.K, args.group
    t = gu.transform_for(wl)
    x0 = gu.x_to_device(wl.x, wl.x_dtype)
    qbytes = M * K * 2 + M * K // 2 + M * (K // grp) * 4
    dbytes = M * K // 2 + M * (K // grp) * 4 + M * K * 2
    nsets = max(2, math.ceil(MALL_FLUSH_BYTES / (qbytes + dbytes)))
    sets = [dict(x=x0.clone(), qa=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                 sa=torch.empty((M, K // grp), dtype=torch.float32, device=dev),
                 out=torch.empty((M, K), dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev).cuda_stream

    if args.launch == "eager":
        def q_only(i):
            st = sets[i % nsets]
            rw4.quantize_act(t, st["x"], "group128", qa=st["qa"], sa=st["sa"], group=grp)

        def d_only(i):
            st = sets[i % nsets]
            rw4.dequantize(st["qa"], st["sa"], out=st["out"])
    else:
        qc = [rw4.prepare_quantize_act(t, st["x"], "group128", qa=st["qa"], sa=st["sa"], group=grp) for st in sets]
        dc = [rw4.prepare_dequantize(st["qa"], st["sa"], out=st["out"]) for st in sets]

        def q_only(i):
            qc[i % nsets]()

        def d_only(i):
            dc[i % nsets]()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        q_only(i)
        if ev is not None:
            ev[1].record(stream)
        d_only(i)
        if ev is not None:
            ev[2].record(stream)

    graph = args.launch == "graph"
    if graph:
        graphs = capture_steps(torch, step, nsets)

        def run(i, ev=None):  # the whole step, one graph launch
            if ev is not None:
                ev[0].record(stream)
            graphs[i % nsets].replay()
            if ev is not None:
                ev[2].record(stream)
    else:
        run = step

    warm = warm_up(run, args, torch)
    # the kernels' durations come from the back-to-back runs below; the timed region is
    # bracketed as a whole (events around each short launch would slow the host further)
    r0, r1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        run(args.warmup + i)
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_gpu_us = 1e3 * r0.elapsed_ms(r1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = (qbytes + dbytes) / (ms_per_step * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us ({'one graph launch' if graph else args.launch + ' calls'}; "
        f"GPU {step_gpu_us:.1f} us)")

    # the kernels run about as long as the host takes per Python call: time them with the host ahead
    (q_b2b, q_ahead), (d_b2b, d_ahead) = gpu_bound_us(torch, stream, q_only), gpu_bound_us(torch, stream, d_only)
    qb_gbps, db_gbps = qbytes / (q_b2b * 1e-6) / 1e9, dbytes / (d_b2b * 1e-6) / 1e9
    log(f"back-to-back (host ahead: {q_ahead and d_ahead}): quantize {q_b2b:.2f} us ({qb_gbps:.0f} GB/s)  "
        f"dequantize {d_b2b:.2f} us ({db_gbps:.0f} GB/s)")
    # the query side: rotate_act (same transform, unquantized bf16 out) over as many query rows
    rbytes = M * K * 2 + M * K * 2
    rc = [rw4.prepare_rotate_act(t, st["x"], out=st["out"]) for st in sets]
    r_b2b, r_ahead = gpu_bound_us(torch, stream, lambda i: rc[i % nsets]())
    rb_gbps = rbytes / (r_b2b * 1e-6) / 1e9
    log(f"rotate_act (queries, bf16 in/out): {r_b2b:.2f} us ({rb_gbps:.0f} GB/s, host ahead: {r_ahead})")
    out = {
        "metric": KV_METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_run": warm, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in/out, int4 codes, fp32 transform and scales", "data": "synthetic",
        "config": {"workload": f"kv M={M} K={K} (8 heads x 128)", "group": grp, "buffer_sets": nsets,
                   "launch": "one HIP graph replay per step" if graph else args.launch + " calls"},
        "step_gpu_us": step_gpu_us,
        "roofline": {"bound": "hbm", "achieved": qb_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": qb_gbps / PEAK_HBM_GBPS, "traffic": None, "kernel": "quant_h128_act_kernel",
                     "algorithmic_bytes_per_launch": qbytes, "avg_launch_us": q_b2b,
                     "timing": "HIP events around 20 launches queued behind a 1 GiB copy (host ahead: "
                               f"{q_ahead}): the kernel's own duration"},
        "dequantize": {"kernel": "dequant_kernel", "avg_launch_us": d_b2b,
                       "gbps": db_gbps, "frac_hbm": db_gbps / PEAK_HBM_GBPS, "algorithmic_bytes": dbytes,
                       "host_ahead": d_ahead},
        "rotate_queries": {"kernel": "rotate_h128_kernel", "avg_launch_us": r_b2b, "gbps": rb_gbps,
                           "frac_hbm": rb_gbps / PEAK_HBM_GBPS, "algorithmic_bytes": rbytes, "host_ahead": r_ahead},
    }
    out["device"] = device_info(torch)  # the clock as the timed region left it, before the CPU leg
    if not args.no_cpu_baseline:
        import oracle
        from tests.helpers import spec_of
        rows = args.cpu_rows or M
        dt, passes = 0.0, 0
        while dt < 10.0 and passes < 1024:  # repeat the sample for ~10 s of CPU work
            t1 = time.perf_counter()
            a = oracle.quantize_act(wl.x[:rows], spec_of(wl), "group128", grp)
            oracle.round_dequant_output(oracle.dequantize(a["codes"], a["sa"], grp), "bf16")
            dt += time.perf_counter() - t1
            passes += 1
        cpu_bytes = (qbytes + dbytes) * rows / M * passes
        bi = blas_info()
        out["cpu_baseline"] = {"value": cpu_bytes / dt / 1e9, "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
                               "kind": "oracle", "sample": f"{rows} of {M} tokens, {passes} pass(es), quantize_act + "
                                                         f"dequantize (float64 numpy)", "seconds": dt,
                               "os_cpu_count": os.cpu_count(), "blas": bi["library"], "blas_file": bi["file"],
                               "blas_threads": bi["threads"]}
    emit(out, torch)


def main_rrs_reorder(args, torch, rw4, gu, dev):
    """Rotated Runtime Smooth with the channel reorder on the RRS workload: one step =
    quantize_act_rrs_reorder (four kernels: channel maxima, their reduction, the order
    and group scales, the reordered quantizer) + permute_codes of the per-channel weights
    by that order + w4a4_gemm."""
    import datagen
    wl = datagen.make("rrs")
    M, K, N = wl.M, wl.K, wl.N
    t = gu.transform_for(wl)
    x = gu.x_to_device(wl.x, wl.x_dtype)
    w = torch.from_numpy(wl.w).to(dev)
    qw, sw = rw4.pack_weight_per_channel(t, w)
    del w
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    order = torch.empty((K,), dtype=torch.int32, device=dev)
    ws = torch.empty((int(rw4.lib.rw4_rrs_reorder_workspace_bytes(K)),), dtype=torch.uint8, device=dev)
    qw_ord = torch.empty_like(qw)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    perm = rw4.prepare_permute_codes(qw, order, out=qw_ord)
    gemm = rw4.prepare_w4a4_gemm(qa, sa, qw_ord, sw, out=y)

    def q_call(i):
        rw4.quantize_act_rrs_reorder(t, x, qa=qa, sa=sa, order=order, workspace=ws)

    def step(i):
        q_call(i)
        perm()
        gemm()

    warm = warm_up(step, args, torch)
    r0, r1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    (q_us, _), (p_us, _), (g_us, _) = (gpu_bound_us(torch, stream, q_call), gpu_bound_us(torch, stream, lambda i: perm()),
                                       gpu_bound_us(torch, stream, lambda i: gemm()))
    ops = 2.0 * M * N * K
    qbytes = M * K * 2 * 2 + M * K // 2 + M * (K // 128) * 4  # X read by both passes, codes and scales written
    pbytes = 2 * N * K // 2
    log(f"rrs reorder step {ms_per_step * 1e3:.1f} us: quantize (4 kernels) {q_us:.2f} us, weight permutation "
        f"{p_us:.2f} us ({pbytes / p_us / 1e3:.0f} GB/s), gemm {g_us:.2f} us ({ops / g_us / 1e6:.0f} TOPS)")
    out = {"metric": METRIC, "value": ops / (ms_per_step * 1e-3) / 1e12, "unit": "TOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "warmup_run": warm, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "int4 codes (exact on fp6 MFMA), fp32 transform, rescale and epilogue", "data": "synthetic",
           "config": {"workload": f"rrs_reorder M={M} K={K} N={N}", "transform": f"hadamard{K}",
                      "act_mode": "rrs with channel reorder", "weights": "per output channel, permuted per call"},
           "quantize_us": q_us, "permute_us": p_us, "gemm_us": g_us,
           "roofline": {"bound": "mfma", "achieved": ops / g_us / 1e6, "peak": PEAK_I8_TOPS, "unit": "TFLOP/s",
                        "frac": ops / g_us / 1e6 / PEAK_I8_TOPS, "peak_fp6": PEAK_F6_TFLOPS,
                        "frac_fp6": ops / g_us / 1e6 / PEAK_F6_TFLOPS, "traffic": None, "kernel": "gemm_f8p_kernel",
                        "avg_launch_us": g_us},
           "permute": {"kernel": "permute_codes_kernel", "avg_launch_us": p_us, "algorithmic_bytes": pbytes,
                       "gbps": pbytes / p_us / 1e3, "frac_hbm": pbytes / p_us / 1e3 / PEAK_HBM_GBPS},
           "quantize": {"kernels": "rrs_chanmax + chanmax_reduce + rrs_rank + quant_rrs_order", "avg_us": q_us,
                        "algorithmic_bytes": qbytes, "gbps": qbytes / q_us / 1e3}}
    emit(out, torch)


def main_decode_fused(args, torch, rw4, gu, dev):
    """One decode step in one launch (decode_fused: quantize inside the small-M GEMM) on the
    decode shape with the block-128 Hadamard, M = 1..16 tokens, against the two launches
    (quantize_act + w4a4_gemm) it replaces."""
    import datagen
    M = int(args.workload[len("fused"):])
    wl = datagen.make("decode", M=M)
    K, N = wl.K, wl.N
    t = rw4.Transform.hadamard(K, 128)
    x = gu.x_to_device(wl.x, wl.x_dtype)
    qw0, sw0 = rw4.pack_weight(t, torch.from_numpy(wl.w).to(dev))
    nsets = max(2, math.ceil(MALL_FLUSH_BYTES / (N * K // 2 + N * K // 32)))
    sets = [(qw0.clone(), sw0.clone(), torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    fused = [rw4.prepare_decode_fused(t, x, q, s, out=y) for q, s, y in sets]
    qc = rw4.prepare_quantize_act(t, x, qa=qa, sa=sa)
    gc = [rw4.prepare_w4a4_gemm(qa, sa, q, s, out=y) for q, s, y in sets]
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(i):
        fused[i % nsets]()

    def two(i):
        qc()
        gc[i % nsets]()

    def step_and_two(i):
        step(i)
        two(i)

    warm = warm_up(step_and_two, args, torch)
    r0, r1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    (f_us, f_ok), (t_us, t_ok) = gpu_bound_us(torch, stream, step, reps=40), gpu_bound_us(torch, stream, two, reps=40)
    ops = 2.0 * M * N * K
    hbm = M * K * 2 + N * K // 2 + N * (K // 128) * 4 + M * N * 2  # x, weights, scales, y
    log(f"decode_fused M={M} K={K} N={N}: {f_us:.2f} us per step back to back (host ahead {f_ok}); "
        f"quantize_act + w4a4_gemm {t_us:.2f} us (host ahead {t_ok})")
    out = {"metric": METRIC, "value": ops / (ms_per_step * 1e-3) / 1e12, "unit": "TOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "warmup_run": warm, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "int4 codes (exact on fp6 MFMA), fp32 transform, rescale and epilogue", "data": "synthetic",
           "config": {"workload": f"decode_fused M={M} K={K} N={N}", "transform": "hadamard128",
                      "act_mode": "group128"},
           "fused_us": f_us, "two_launch_us": t_us,
           "roofline": {"bound": "hbm", "achieved": hbm / f_us / 1e3, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": hbm / f_us / 1e3 / PEAK_HBM_GBPS, "traffic": None, "kernel": "decode_fused_kernel",
                        "avg_launch_us": f_us, "algorithmic_bytes": hbm}}
    emit(out, torch)


def main_asym(args, torch, rw4, gu, dev):
    """Asymmetric (s, z) activations on a block-128 Hadamard workload: one step =
    quantize_act_asym + w4a4_gemm_asym (weights and their code sums packed offline),
    beside the symmetric step on the same data."""
    base = args.workload[:-len("_asym")]
    wl = workload(base)
    M, K, N = wl.M, wl.K, wl.N
    G = K // 128
    t = rw4.Transform.hadamard(K, 128)
    x0 = gu.x_to_device(wl.x, wl.x_dtype)
    qw0, sw0 = rw4.pack_weight(t, torch.from_numpy(wl.w).to(dev))
    cw0 = rw4.weight_code_sums(qw0)
    set_bytes = M * K * 2 + M * K // 2 + 2 * M * G * 4 + N * K // 2 + 2 * N * G * 4 + M * N * 2
    nsets = max(2, math.ceil(MALL_FLUSH_BYTES / set_bytes))
    sets = []
    for _ in range(nsets):
        sets.append(dict(x=x0.clone(), qa=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                         sa=torch.empty((M, G), dtype=torch.float32, device=dev),
                         za=torch.empty((M, G), dtype=torch.float32, device=dev),
                         qw=qw0.clone(), sw=sw0.clone(), cw=cw0.clone(),
                         y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    qc = [rw4.prepare_quantize_act_asym(t, s["x"], qa=s["qa"], sa=s["sa"], za=s["za"]) for s in sets]
    gc = [rw4.prepare_w4a4_gemm_asym(s["qa"], s["sa"], s["za"], s["qw"], s["sw"], s["cw"], out=s["y"]) for s in sets]
    qs = [rw4.prepare_quantize_act(t, s["x"], qa=s["qa"], sa=s["sa"]) for s in sets]
    gs = [rw4.prepare_w4a4_gemm(s["qa"], s["sa"], s["qw"], s["sw"], out=s["y"]) for s in sets]
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(i):
        qc[i % nsets]()
        gc[i % nsets]()

    warm = warm_up(step, args, torch)
    r0, r1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    (q_us, _), (g_us, _) = (gpu_bound_us(torch, stream, lambda i: qc[i % nsets]()),
                            gpu_bound_us(torch, stream, lambda i: gc[i % nsets]()))
    (qs_us, _), (gs_us, _) = (gpu_bound_us(torch, stream, lambda i: qs[i % nsets]()),
                              gpu_bound_us(torch, stream, lambda i: gs[i % nsets]()))
    ops = 2.0 * M * N * K
    qbytes = M * K * 2 + M * K // 2 + 2 * M * G * 4
    gk = gemm_kernel_for(M, N)
    log(f"{args.workload} M={M} K={K} N={N}: step {ms_per_step * 1e3:.1f} us; asymmetric quantize {q_us:.2f} us, "
        f"gemm {g_us:.2f} us ({ops / g_us / 1e6:.0f} TOPS); symmetric quantize {qs_us:.2f} us, gemm {gs_us:.2f} us")
    out = {"metric": METRIC, "value": ops / (ms_per_step * 1e-3) / 1e12, "unit": "TOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "warmup_run": warm, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "int4 codes (exact on fp6 MFMA), fp32 transform, rescale and epilogue", "data": "synthetic",
           "config": {"workload": f"{args.workload} M={M} K={K} N={N}", "transform": "hadamard128",
                      "act_mode": "group128 asymmetric (s, z)"},
           "quantize_us": q_us, "gemm_us": g_us, "symmetric_quantize_us": qs_us, "symmetric_gemm_us": gs_us,
           "roofline": {"bound": "mfma", "achieved": ops / g_us / 1e6, "peak": PEAK_I8_TOPS, "unit": "TFLOP/s",
                        "frac": ops / g_us / 1e6 / PEAK_I8_TOPS, "peak_fp6": PEAK_F6_TFLOPS,
                        "frac_fp6": ops / g_us / 1e6 / PEAK_F6_TFLOPS, "traffic": None, "kernel": gk, "avg_launch_us": g_us},
           "quantize": {"kernel": "quant_h128_act_kernel (asymmetric)", "avg_us": q_us, "algorithmic_bytes": qbytes,
                        "gbps": qbytes / q_us / 1e3, "frac_hbm": qbytes / q_us / 1e3 / PEAK_HBM_GBPS}}
    emit(out, torch)


def main_mixed(args, torch, rw4, gu, dev, n8=4):
    """8-bit groups for extreme outliers on a block-128 Hadamard workload: the n8 groups
    holding the workload's largest channel maxima are kept at 8 bits (two INT4 planes); one
    step = quantize_act_mixed + w4a4_gemm over K + 128 n8 (weights extended offline), beside
    the all-INT4 step on the same data."""
    base = args.workload[:-len("_mixed")]
    wl = workload(base)
    M, K, N = wl.M, wl.K, wl.N
    G = K // 128
    t = rw4.Transform.hadamard(K, 128)
    gmax = np.abs(wl.x).reshape(M, G, 128).max(axis=(0, 2))
    groups8 = sorted(int(g) for g in np.argsort(-gmax)[:n8])
    slot, glist = rw4.mixed_tables(K, groups8, dev)
    x = gu.x_to_device(wl.x, wl.x_dtype)
    qw, sw = rw4.pack_weight(t, torch.from_numpy(wl.w).to(dev))
    qx, sx = rw4.extend_weight_groups(qw, sw, glist)
    Kx = K + 128 * n8
    nsets = max(2, math.ceil(MALL_FLUSH_BYTES / (M * K * 2 + M * Kx // 2 + N * Kx // 2 + M * N * 2)))
    sets = []
    for _ in range(nsets):
        sets.append(dict(x=x.clone(), qa=torch.empty((M, Kx // 2), dtype=torch.uint8, device=dev),
                         sa=torch.empty((M, Kx // 128), dtype=torch.float32, device=dev),
                         q4=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                         s4=torch.empty((M, G), dtype=torch.float32, device=dev),
                         qx=qx.clone(), sx=sx.clone(), qw=qw.clone(), sw=sw.clone(),
                         y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
    qc = [rw4.prepare_quantize_act_mixed(t, s["x"], slot, n8, qa=s["qa"], sa=s["sa"]) for s in sets]
    gc = [rw4.prepare_w4a4_gemm(s["qa"], s["sa"], s["qx"], s["sx"], out=s["y"]) for s in sets]
    q4 = [rw4.prepare_quantize_act(t, s["x"], qa=s["q4"], sa=s["s4"]) for s in sets]
    g4 = [rw4.prepare_w4a4_gemm(s["q4"], s["s4"], s["qw"], s["sw"], out=s["y"]) for s in sets]
    stream = torch.cuda.current_stream(dev).cuda_stream

    def step(i):
        qc[i % nsets]()
        gc[i % nsets]()

    warm = warm_up(step, args, torch)
    r0, r1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    (q_us, _), (g_us, _) = (gpu_bound_us(torch, stream, lambda i: qc[i % nsets]()),
                            gpu_bound_us(torch, stream, lambda i: gc[i % nsets]()))
    (q4_us, _), (g4_us, _) = (gpu_bound_us(torch, stream, lambda i: q4[i % nsets]()),
                              gpu_bound_us(torch, stream, lambda i: g4[i % nsets]()))
    ops = 2.0 * M * N * K
    log(f"{args.workload} M={M} K={K} N={N}, 8-bit groups {groups8}: step {ms_per_step * 1e3:.1f} us; "
        f"mixed quantize {q_us:.2f} us, gemm over K + {128 * n8} {g_us:.2f} us; all-INT4 quantize {q4_us:.2f} us, "
        f"gemm {g4_us:.2f} us")
    out = {"metric": METRIC, "value": ops / (ms_per_step * 1e-3) / 1e12, "unit": "TOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "warmup_run": warm, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None,
           "dtype": "int4 codes (exact on fp6 MFMA), fp32 transform, rescale and epilogue", "data": "synthetic",
           "config": {"workload": f"{args.workload} M={M} K={K} N={N}", "transform": "hadamard128",
                      "act_mode": f"group128 with {n8} groups at 8 bits (two INT4 planes)", "groups8": groups8},
           "quantize_us": q_us, "gemm_us": g_us, "int4_quantize_us": q4_us, "int4_gemm_us": g4_us,
           "roofline": {"bound": "mfma", "achieved": ops / g_us / 1e6, "peak": PEAK_I8_TOPS, "unit": "TFLOP/s",
                        "frac": ops / g_us / 1e6 / PEAK_I8_TOPS, "peak_fp6": PEAK_F6_TFLOPS,
                        "frac_fp6": ops / g_us / 1e6 / PEAK_F6_TFLOPS, "traffic": None, "kernel": gemm_kernel_for(M, N),
                        "avg_launch_us": g_us, "note": "ops of the layer (2 M N K), the GEMM runs over K + 128 n8"}}
    emit(out, torch)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path shards "
              "without communication (see the design notes) and no multi-GPU run is made.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import rotated_w4a4_amd as rw4
    from tests import gpu_util as gu

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = args.calibrate_copy * 2**20 // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copied {args.calibrate_copy} MiB x5 ({n * 4} bytes read and written per copy)")
        return
    if args.workload == "kv":
        return main_kv(args, torch, rw4, gu, dev)
    if args.workload == "rrs_reorder":
        return main_rrs_reorder(args, torch, rw4, gu, dev)
    if args.workload.startswith("fused"):
        return main_decode_fused(args, torch, rw4, gu, dev)
    if args.workload.endswith("_asym"):
        return main_asym(args, torch, rw4, gu, dev)
    if args.workload.endswith("_mixed"):
        return main_mixed(args, torch, rw4, gu, dev)
    wl = workload(args.workload)
    M, K, N = wl.M, wl.K, wl.N
    grp = args.group
    if grp != 128 and not (wl.transform == ("hadamard", 128) and wl.mode == "group128"):
        raise SystemExit("--group 64/256 needs a block-128 Hadamard workload in per-group mode")
    G = K // grp
    log(f"workload {wl.name} M={M} K={K} N={N} transform={wl.transform} mode={wl.mode} "
        f"device={torch.cuda.get_device_name(dev)}")

    t = gu.transform_for(wl)
    x0 = gu.x_to_device(wl.x, wl.x_dtype)
    w0 = torch.from_numpy(wl.w).to(dev)
    qw0, sw0 = rw4.pack_weight(t, w0, group=grp)
    torch.cuda.synchronize()
    del w0

    ydt = torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32
    qbytes, gbytes = algorithmic_bytes(wl, grp)
    set_bytes = qbytes + gbytes
    nsets = max(2, math.ceil(MALL_FLUSH_BYTES / set_bytes))
    sets = []
    for _ in range(nsets):
        sets.append(dict(
            x=x0.clone(),
            qa=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
            sa=torch.empty((M, G), dtype=torch.float32, device=dev),
            qw=qw0.clone(), sw=sw0.clone(),
            y=torch.empty((M, N), dtype=ydt, device=dev),
            ws=torch.zeros((max(G, 4),), dtype=torch.float32, device=dev)))
    del x0
    torch.cuda.synchronize()
    log(f"{nsets} rotating buffer sets of {set_bytes / 2**20:.1f} MiB")

    stream = torch.cuda.current_stream(dev).cuda_stream  # the stream the kernels run on

    if args.launch == "eager":
        def q_call(i):
            s = sets[i % nsets]
            rw4.quantize_act(t, s["x"], wl.mode, qa=s["qa"], sa=s["sa"], workspace=s["ws"], group=grp)

        def g_call(i):
            s = sets[i % nsets]
            rw4.w4a4_gemm(s["qa"], s["sa"], s["qw"], s["sw"], out=s["y"])
    else:
        qc = [rw4.prepare_quantize_act(t, s["x"], wl.mode, qa=s["qa"], sa=s["sa"], workspace=s["ws"], group=grp)
              for s in sets]
        gc = [rw4.prepare_w4a4_gemm(s["qa"], s["sa"], s["qw"], s["sw"], out=s["y"]) for s in sets]

        def q_call(i):
            qc[i % nsets]()

        def g_call(i):
            gc[i % nsets]()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        q_call(i)
        if ev is not None:
            ev[1].record(stream)
        g_call(i)
        if ev is not None:
            ev[2].record(stream)

    graph = args.launch == "graph"
    if graph:
        graphs = capture_steps(torch, step, nsets)

        def run(i, ev=None):  # the whole step, one graph launch
            if ev is not None:
                ev[0].record(stream)
            graphs[i % nsets].replay()
            if ev is not None:
                ev[2].record(stream)
    else:
        run = step

    warm = warm_up(run, args, torch)

    # timed region: exactly `steps` steps, events on the launch stream.  Every EVENT_EVERY-th
    # step records events around its two kernels: recording them on every step adds ~4.4 us
    # per q_proj step (measured), which would slow the very throughput being timed.
    # Decode-sized steps take the kernels' durations from the back-to-back runs below
    # (events around each of their launches would count host gaps), so only the whole
    # region is bracketed there.
    decode = M <= 64  # the small-M GEMM: weights streamed once, below the MFMA ridge point
    per_step = not decode and not graph
    events = [[HipEvent() for _ in range(3)] if per_step and i % EVENT_EVERY == 0 else None
              for i in range(args.steps)]
    r0, r1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        run(args.warmup + i, events[i])
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ops = 2.0 * M * N * K
    step_gpu_us = 1e3 * r0.elapsed_ms(r1) / args.steps
    q_spread = g_spread = None
    if per_step:
        q_list = [1e3 * e[0].elapsed_ms(e[1]) for e in events if e]
        g_list = [1e3 * e[1].elapsed_ms(e[2]) for e in events if e]
        q_us, g_us = float(np.mean(q_list)), float(np.mean(g_list))
        q_spread, g_spread = spread(q_list), spread(g_list)
    else:
        q_us = g_us = float("nan")  # replaced by the back-to-back times below
    layer_tops = ops / (ms_per_step * 1e-3) / 1e12

    # each kernel alone, launched back to back behind a copy that lets the host run ahead
    (q_b2b, q_ahead), (g_b2b, g_ahead) = gpu_bound_us(torch, stream, q_call), gpu_bound_us(torch, stream, g_call)
    log(f"back-to-back (host ahead: {q_ahead and g_ahead}): quantize {q_b2b:.2f} us, gemm {g_b2b:.2f} us")
    if not per_step:  # per-kernel times: the kernels alone, back to back
        q_us, g_us = q_b2b, g_b2b
    gemm_tops = ops / (g_us * 1e-6) / 1e12
    quant_gbps = qbytes / (q_us * 1e-6) / 1e9
    gemm_gbps = gbytes / (g_us * 1e-6) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us ({'one graph launch' if graph else args.launch + ' calls'}; "
        f"GPU {step_gpu_us:.1f} us)  quantize {q_us:.2f} us ({quant_gbps:.0f} GB/s)  "
        f"gemm {g_us:.2f} us ({gemm_tops:.0f} TOPS)")

    gemm_kernel = gemm_kernel_for(M, N, grp)
    wkey = args.workload if grp == 128 else f"{args.workload}_g{grp}"  # counters are per configuration
    traffic = measured_traffic(gemm_kernel, wkey)
    if decode:
        # the small-M GEMM streams the packed weights: HBM-bound.  A decode step is shorter than
        # the host's two Python calls, so events around each launch in the step also count the
        # GPU waiting for the host; the kernel's own rate is the back-to-back one.
        b2b_gbps = gbytes / (g_b2b * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": b2b_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": b2b_gbps / PEAK_HBM_GBPS, "traffic": traffic,
                "kernel": gemm_kernel, "algorithmic_bytes_per_launch": gbytes,
                "avg_launch_us": g_b2b,
                "timing": "HIP events around 20 launches queued behind a 1 GiB copy (host ahead: "
                          f"{g_ahead}): the kernel's own duration, which events around one launch of an "
                          "eager step overstate by the host's launch gaps"}
    else:
        roof = {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_I8_TOPS, "unit": "TFLOP/s",
                "frac": gemm_tops / PEAK_I8_TOPS, "peak_fp6": PEAK_F6_TFLOPS, "frac_fp6": gemm_tops / PEAK_F6_TFLOPS,
                "traffic": traffic,
                "kernel": gemm_kernel, "ops_per_launch": ops, "avg_launch_us": g_us,
                "algorithmic_bytes_per_launch": gbytes,
                "note": "ops = 2 M N K (2 per MAC of INT4 codes, computed exactly on the FP6 MFMA) against the dense int8 MFMA peak (frac) and the dense FP6 peak (frac_fp6); traffic in bytes"}
    if wl.transform[0] == "givens":
        quant_kernel = "quant_givens_kernel"
    elif wl.transform[1] == 128 and wl.mode == "group128":
        quant_kernel = "quant_h128_act_kernel"
    elif wl.mode == "rrs" and wl.transform[1] == K and K in (2048, 4096, 8192) and wl.signs is None:
        quant_kernel = "quant_rrs_full_kernel"  # after rrs_colmax_full_kernel, in the same call
    else:
        quant_kernel = "quant_rowh_kernel"
    out = {
        "metric": METRIC,
        "value": layer_tops,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes (exact on fp6 MFMA), fp32 transform, rescale and epilogue",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} M={M} K={K} N={N}", "M": M, "K": K, "N": N,
                   "transform": f"{wl.transform[0]}{wl.transform[1]}", "act_mode": wl.mode,
                   "x_dtype": wl.x_dtype, "y_dtype": wl.y_dtype, "weights": "packed offline",
                   "buffer_sets": nsets, "group": grp,
                   "launch": "one HIP graph replay per step" if graph else args.launch + " calls"},
        "roofline": roof,
        "quantize": {"kernel": quant_kernel, "avg_launch_us": q_us, "launch_us": q_spread, "gbps": quant_gbps,
                     "frac_hbm": quant_gbps / PEAK_HBM_GBPS, "algorithmic_bytes": qbytes,
                     "back_to_back_us": q_b2b, "back_to_back_gbps": qbytes / (q_b2b * 1e-6) / 1e9,
                     "back_to_back_host_ahead": q_ahead,
                     "back_to_back_frac_hbm": qbytes / (q_b2b * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     "traffic": measured_traffic(quant_kernel, wkey)},
        "gemm": {"kernel": gemm_kernel, "avg_launch_us": g_us, "launch_us": g_spread, "tops": gemm_tops,
                 "frac_mfma": gemm_tops / PEAK_I8_TOPS, "gbps": gemm_gbps,
                 "back_to_back_us": g_b2b, "back_to_back_tops": ops / (g_b2b * 1e-6) / 1e12,
                 "back_to_back_gbps": gbytes / (g_b2b * 1e-6) / 1e9, "back_to_back_host_ahead": g_ahead},
        "layer_us": ms_per_step * 1e3,
        "step_gpu_us": step_gpu_us,
        "instrumented_steps": sum(1 for e in events if e),
    }
    out["device"] = device_info(torch)  # the clock as the timed region left it, before the CPU leg

    if not args.no_cpu_baseline:
        rows = args.cpu_rows or (M if M <= 64 else max(16, min(M, 256 * 4096 // K)))
        dt, threads = cpu_baseline(wl, rows)
        if dt < 5.0 and rows < M:  # aim for 10-30 s of CPU work
            rows = min(M, int(rows * 12.0 / max(dt, 1e-3)))
            dt, threads = cpu_baseline(wl, rows)
        passes = 1
        while dt < 10.0 and passes < 64:  # the whole sample is quick: repeat it for ~10 s
            more, threads = cpu_baseline(wl, rows)
            dt += more
            passes += 1
        cpu_tops = 2.0 * rows * N * K * passes / dt / 1e12
        bi = blas_info()
        out["cpu_baseline"] = {"value": cpu_tops, "unit": "TOPS", "cores": threads, "kind": "oracle",
                               "sample": f"{rows} of {M} tokens of the same layer, {passes} pass(es), quantize_act + "
                                         f"w4a4_gemm (float64 numpy), weights packed beforehand",
                               "seconds": dt, "host_cpus": len(os.sched_getaffinity(0)),
                               "os_cpu_count": os.cpu_count(), "blas": bi["library"], "blas_file": bi["file"],
                               "blas_threads": bi["threads"]}
        log(f"cpu oracle: {passes} x {rows} rows in {dt:.2f} s = {cpu_tops * 1e3:.3f} GOPS on {threads} threads")
    emit(out, torch)


if __name__ == "__main__":
    main()
