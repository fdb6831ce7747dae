"""Helpers for the GPU parity tests: host <-> device transfers of raw bits."""
import numpy as np
import torch

DEV = "cuda:0"


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def fp8_to_dev(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).to(DEV).view(torch.float8_e4m3fn)


def fp8_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def announce(*parts):
    """Name the case on stdout before GPU work (a faulting run leaves this)."""
    print("CASE", *parts, flush=True)
