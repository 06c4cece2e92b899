"""Host <-> device plumbing shared by the GPU tests (no method arithmetic)."""

import sys

import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(bits):
    """uint16 BF16 bit patterns (numpy) -> torch.bfloat16 on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16).to(dev())


def to_dev(arr, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def host(t):
    """Device tensor -> numpy (bfloat16 comes back as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()
