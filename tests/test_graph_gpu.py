"""Launch paths of the hot path: HIP graph capture and prepared calls.

quantize_act + w4a4_gemm only launch kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a serving loop can record a
step once into a graph and replay it, paying one graph launch on the host
instead of two Python calls.  Each case records the step on torch's capture
stream, then replays it several times with new inputs copied into the
recorded input buffer and unrelated eager work and synchronisations between
the replays; every replay must equal, bit for bit, the eager calls on the
same input (the same kernels run on the same data).
"""
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402

if torch.cuda.is_available():
    import rotated_w4a4_amd as rw4  # noqa: E402
    from tests import gpu_util as gu  # noqa: E402

CASES = [
    # name, workload, overrides: the decode step (Givens layers, small-M GEMM), a prefill
    # q_proj slice (block-128 Hadamard, tiled GEMM), Rotated Runtime Smooth (two passes and
    # a fill kernel on the workspace)
    ("decode16_givens", "decode", dict(M=16, K=1024, N=512)),
    ("q_proj_h128", "q_proj", dict(M=300, K=1024, N=384)),
    ("rrs_full_row", "rrs", dict(M=200, K=2048, N=256)),
]


def _inputs(x0):
    """Three distinct inputs of the same shape whose values stay exact in bf16."""
    return [x0, torch.roll(x0, 7, dims=0) * 2.0, torch.roll(x0, -3, dims=0) * 0.5]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(case):
    name, kind, kw = case
    print(f"graph case {name}", flush=True)
    wl = datagen.make(kind, seed=11, **kw)
    t = gu.transform_for(wl)
    qw, sw = rw4.pack_weight(t, torch.from_numpy(wl.w).to(gu.DEV))
    x0 = gu.x_to_device(wl.x, wl.x_dtype)
    M, K, N = wl.M, wl.K, wl.N
    G = K // 128

    def buffers():
        return dict(qa=torch.empty((M, K // 2), dtype=torch.uint8, device=gu.DEV),
                    sa=torch.empty((M, G), dtype=torch.float32, device=gu.DEV),
                    ws=torch.zeros((max(G, 4),), dtype=torch.float32, device=gu.DEV),
                    y=torch.empty((M, N), dtype=torch.bfloat16, device=gu.DEV))

    def step(x, b):
        rw4.quantize_act(t, x, wl.mode, qa=b["qa"], sa=b["sa"], workspace=b["ws"])
        rw4.w4a4_gemm(b["qa"], b["sa"], qw, sw, out=b["y"])

    xs = _inputs(x0)
    refs = []
    for x in xs:  # eager results, each in buffers of its own
        b = buffers()
        step(x, b)
        refs.append(b)
    torch.cuda.synchronize()

    x_static = x0.clone()
    bs = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager run on a side stream before capture
        step(x_static, bs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x_static, bs)
    torch.cuda.synchronize()

    noise_a = torch.randn((512, 512), device=gu.DEV)
    for rep in range(2):
        for k, x in enumerate(xs):
            x_static.copy_(x)
            _ = noise_a @ noise_a  # unrelated eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for key in ("qa", "sa", "y"):
                assert torch.equal(bs[key], refs[k][key]), f"{name}: replay {rep}/{k} differs in {key}"


def _replays_match(name, step, buffers, xs, keys):
    """Record step(x_static, b) into a graph; every replay on each input of
    xs must equal, bit for bit, eager calls on that input."""
    refs = []
    for x in xs:
        b = buffers()
        step(x, b)
        refs.append(b)
    torch.cuda.synchronize()
    x_static = xs[0].clone()
    bs = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(x_static, bs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x_static, bs)
    torch.cuda.synchronize()
    noise_a = torch.randn((512, 512), device=gu.DEV)
    for rep in range(2):
        for k, x in enumerate(xs):
            x_static.copy_(x)
            _ = noise_a @ noise_a
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for key in keys:
                assert torch.equal(bs[key], refs[k][key]), f"{name}: replay {rep}/{k} differs in {key}"


NEWER = ["decode_fused_m4", "asym_q_proj", "rrs_reorder", "mixed_q_proj"]


@pytest.mark.parametrize("name", NEWER)
def test_graph_replays_newer_entry_points(name):
    """The same check for the one-launch decode step, the asymmetric pair, the
    RRS reorder pipeline (order, its workspace, the weight permutation) and
    the 8-bit-group pair: none of them allocates, clears memory with a
    memset or synchronises, so each records into a graph and replays."""
    print(f"graph case {name}", flush=True)
    E = dict(dtype=torch.bfloat16, device=gu.DEV)
    if name == "rrs_reorder":
        wl = datagen.make("rrs", seed=15, M=200, K=2048, N=256)
    else:
        wl = datagen.make("q_proj", seed=13, M=4 if name == "decode_fused_m4" else 300, K=1024,
                          N=512 if name == "decode_fused_m4" else 384)
    t = gu.transform_for(wl)
    M, K, N = wl.M, wl.K, wl.N
    G = K // 128
    w = torch.from_numpy(wl.w).to(gu.DEV)
    xs = _inputs(gu.x_to_device(wl.x, wl.x_dtype))
    u8 = dict(dtype=torch.uint8, device=gu.DEV)
    f32 = dict(dtype=torch.float32, device=gu.DEV)
    if name == "decode_fused_m4":
        qw, sw = rw4.pack_weight(t, w)

        def buffers():
            return dict(y=torch.empty((M, N), **E))

        def step(x, b):
            rw4.decode_fused(t, x, qw, sw, out=b["y"])
        keys = ("y",)
    elif name == "asym_q_proj":
        qw, sw = rw4.pack_weight(t, w)
        cw = rw4.weight_code_sums(qw)

        def buffers():
            return dict(qa=torch.empty((M, K // 2), **u8), sa=torch.empty((M, G), **f32),
                        za=torch.empty((M, G), **f32), y=torch.empty((M, N), **E))

        def step(x, b):
            rw4.quantize_act_asym(t, x, qa=b["qa"], sa=b["sa"], za=b["za"])
            rw4.w4a4_gemm_asym(b["qa"], b["sa"], b["za"], qw, sw, cw, out=b["y"])
        keys = ("qa", "sa", "za", "y")
    elif name == "rrs_reorder":
        qw, sw = rw4.pack_weight_per_channel(t, w)
        nbytes = int(rw4.lib.rw4_rrs_reorder_workspace_bytes(K))

        def buffers():
            return dict(qa=torch.empty((M, K // 2), **u8), sa=torch.empty((M, G), **f32),
                        order=torch.empty((K,), dtype=torch.int32, device=gu.DEV),
                        ws=torch.empty((nbytes,), **u8), qw=torch.empty_like(qw), y=torch.empty((M, N), **E))

        def step(x, b):
            rw4.quantize_act_rrs_reorder(t, x, qa=b["qa"], sa=b["sa"], order=b["order"], workspace=b["ws"])
            rw4.permute_codes(qw, b["order"], out=b["qw"])
            rw4.w4a4_gemm(b["qa"], b["sa"], b["qw"], sw, out=b["y"])
        keys = ("qa", "sa", "order", "qw", "y")
    else:
        qw, sw = rw4.pack_weight(t, w)
        slot, glist = rw4.mixed_tables(K, [1, 5], gu.DEV)
        qx, sx = rw4.extend_weight_groups(qw, sw, glist)
        Kx = K + 2 * 128

        def buffers():
            return dict(qa=torch.empty((M, Kx // 2), **u8), sa=torch.empty((M, Kx // 128), **f32),
                        y=torch.empty((M, N), **E))

        def step(x, b):
            rw4.quantize_act_mixed(t, x, slot, 2, qa=b["qa"], sa=b["sa"])
            rw4.w4a4_gemm(b["qa"], b["sa"], qx, sx, out=b["y"])
        keys = ("qa", "sa", "y")
    _replays_match(name, step, buffers, xs, keys)


def test_prepared_calls_match_eager():
    """Calls prepared once (arguments checked and marshalled once) and run
    repeatedly on new contents of the same buffers give the eager results
    bit for bit; each returns the buffers it writes."""
    wl = datagen.make("decode", seed=12, M=16, K=1024, N=512)
    t = gu.transform_for(wl)
    qw, sw = rw4.pack_weight(t, torch.from_numpy(wl.w).to(gu.DEV))
    x0 = gu.x_to_device(wl.x, wl.x_dtype)
    M, K, N = wl.M, wl.K, wl.N
    x_static = torch.empty_like(x0)
    qa = torch.empty((M, K // 2), dtype=torch.uint8, device=gu.DEV)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=gu.DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=gu.DEV)
    xd = torch.empty((M, K), dtype=torch.bfloat16, device=gu.DEV)
    q_call = rw4.prepare_quantize_act(t, x_static, wl.mode, qa=qa, sa=sa)
    g_call = rw4.prepare_w4a4_gemm(qa, sa, qw, sw, out=y)
    d_call = rw4.prepare_dequantize(qa, sa, out=xd)
    for k, x in enumerate(_inputs(x0)):
        qa_ref, sa_ref = rw4.quantize_act(t, x, wl.mode)
        y_ref = rw4.w4a4_gemm(qa_ref, sa_ref, qw, sw, torch.bfloat16)
        xd_ref = rw4.dequantize(qa_ref, sa_ref, torch.bfloat16)
        x_static.copy_(x)
        ret = q_call()
        assert ret[0] is qa and ret[1] is sa and g_call() is y and d_call() is xd
        torch.cuda.synchronize()
        for name, got, ref in (("qa", qa, qa_ref), ("sa", sa, sa_ref), ("y", y, y_ref), ("xd", xd, xd_ref)):
            assert torch.equal(got, ref), f"input {k}: prepared {name} differs"
