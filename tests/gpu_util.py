"""Marshalling helpers for the GPU parity tests: move seeded inputs to the
device, call the library through its binding, bring results back."""
import numpy as np
import torch

import rotated_w4a4_amd as rw4

DEV = "cuda:0"


def x_to_device(x64: np.ndarray, dtype: str):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32)).to(DEV)
    f = np.ascontiguousarray(x64, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), "not bf16 values"
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def transform_for(wl):
    if wl.transform[0] == "hadamard":
        return rw4.Transform.hadamard(wl.K, int(wl.transform[1]), signs=wl.signs)
    return rw4.Transform.givens(wl.K, wl.pairs, wl.theta, wl.beta)


def to_np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def quantize(t, x_dev, mode):
    ws = None
    if mode == "rrs":
        ws = torch.zeros(x_dev.shape[1] // 128, dtype=torch.float32, device=DEV)
    qa, sa = rw4.quantize_act(t, x_dev, mode, workspace=ws)
    return qa, sa, ws
