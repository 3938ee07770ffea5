"""Helpers shared by the GPU tests: moving seeded bf16 inputs to the device
and back. No arithmetic of the method lives here."""
import sys

import numpy as np
import torch

import workloads


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 tensor on cuda:0 (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


class DevInputs:
    def __init__(self, inp: workloads.Inputs):
        self.q = to_dev(inp.q)
        self.k = to_dev(inp.k)
        self.v = to_dev(inp.v)
        self.w_q = f32_dev(inp.w_q)
        self.w_k = f32_dev(inp.w_k)
