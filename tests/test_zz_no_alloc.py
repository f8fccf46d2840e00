"""The allocation-free entry point rw4_quantize_act_static against
rw4_quantize_act (caller workspace): identical codes and scales, bit for bit,
on two calls in a row, the second with a smaller input (the static scratch
keeps the first call's group maxima and must be cleared by the call)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import datagen  # noqa: E402

if torch.cuda.is_available():
    import rotated_w4a4_amd as rw4  # noqa: E402
    from tests import gpu_util as gu  # noqa: E402


def _x(seed, M, K):
    rng = np.random.default_rng(seed)
    return gu.x_to_device(datagen.round_to_bf16(datagen.outlier_activations(rng, M, K)), "bf16")


def _both(t, x, mode):
    ws = torch.full((x.shape[1] // 128,), -1.0, dtype=torch.float32, device=gu.DEV)
    qa1, sa1 = rw4.quantize_act(t, x, mode, workspace=ws)
    qa2, sa2 = rw4.quantize_act_static(t, x, mode)
    torch.cuda.synchronize()
    return (qa1, sa1), (qa2, sa2)


def test_static_scratch_matches_workspace_two_calls():
    # first call: the largest RRS row (K = 8192 fills all 64 scratch floats),
    # second: fewer rows and channels (K = 2048 uses 16 of them)
    for seed, M, K in ((1, 300, 8192), (2, 37, 2048)):
        t = rw4.Transform.hadamard(K, K)
        x = _x(seed, M, K)
        (qa1, sa1), (qa2, sa2) = _both(t, x, "rrs")
        assert torch.equal(qa1, qa2), (M, K)
        assert torch.equal(sa1, sa2), (M, K)
    # a row-transform RRS case (block 1024 < K) and the per-group mode
    t = rw4.Transform.hadamard(4096, 1024)
    (qa1, sa1), (qa2, sa2) = _both(t, _x(3, 20, 4096), "rrs")
    assert torch.equal(qa1, qa2) and torch.equal(sa1, sa2)
    t = rw4.Transform.hadamard(1024, 128)
    (qa1, sa1), (qa2, sa2) = _both(t, _x(4, 9, 1024), "group128")
    assert torch.equal(qa1, qa2) and torch.equal(sa1, sa2)


def test_static_scratch_rejects_and_empty():
    t = rw4.Transform.hadamard(512, 512)
    qa, sa = rw4.quantize_act_static(t, torch.zeros((0, 512), dtype=torch.bfloat16, device=gu.DEV), "rrs")
    assert qa.shape == (0, 256)
    big = rw4.Transform.hadamard(16384, 128)  # K / 128 = 128 > the 64-float scratch
    with pytest.raises(rw4.RW4Error, match="SHAPE"):
        rw4.quantize_act_static(big, torch.zeros((2, 16384), dtype=torch.bfloat16, device=gu.DEV), "rrs")
