"""Shared helpers of the GPU tests: uploads and a progress line per case."""
import sys

import numpy as np
import torch


def say(msg):
    """Name the case before a GPU step, flushed, so a failing run shows where it was."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def to_gpu_bf16(bits):
    """Upload uint16 bf16 bit patterns as a torch bfloat16 GPU tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_gpu_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bf16_bits(t):
    """A bf16 torch tensor's bit patterns as uint16 numpy."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
