"""Helpers shared by the GPU parity tests: moving numpy arrays holding raw
bf16 / e4m3 bit patterns to and from the device, and announcing each case
before it runs (so that a failing run names its case)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*parts):
    print("[case]", *parts, file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(DEV)


def f32_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_host_f64(t: torch.Tensor) -> np.ndarray:
    b = bf16_host(t).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()
