"""Helpers for the GPU tests: move the generators' numpy arrays to the device
and back without touching their bits."""
import numpy as np
import pytest

import workloads as wl


def torch_mod():
    import torch
    return torch


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def require_gpu():
    if not gpu_available():
        pytest.skip("no GPU in this process")


def act_dtype(dtype):
    torch = torch_mod()
    return torch.float16 if dtype == wl.F16 else torch.bfloat16


def dev_act(bits, dtype):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(act_dtype(dtype))
    return t.cuda()


def dev(a):
    torch = torch_mod()
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t):
    torch = torch_mod()
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def w4a16_to_device(d):
    return dict(x=dev_act(d["x"], d["dtype"]), qweight=dev(d["qweight"]),
                scales=dev_act(d["scales"], d["dtype"]), qzeros=dev(d["qzeros"]))


def is_nan_bits(bits, dtype):
    bits = np.asarray(bits, np.uint16)
    if dtype == wl.F16:
        return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x03FF) != 0)
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)
