"""Helpers for the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def u32(t):
    """Host value of a device uint32 scalar held in an int32 tensor."""
    return int(host(t).astype(np.int64).reshape(-1)[0]) & 0xFFFFFFFF


def say(*a):
    print(*a, flush=True)
