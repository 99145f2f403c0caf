"""Host <-> device helpers for the GPU tests (no computation)."""

import sys

import numpy as np
import torch

from synthetic import bf16_bits


def say(*args):
    """Print and flush a line naming the case about to run on the GPU."""
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(a.astype(np.float32))
    elif dtype == "i32":
        t = torch.from_numpy(a.astype(np.int32))
    elif dtype == "u8":
        t = torch.from_numpy(a.astype(np.uint8))
    else:
        raise ValueError(dtype)
    return t.cuda()


def to_host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()
