"""Helpers for the GPU tests: move seeded numpy inputs to the device and back."""
import numpy as np
import torch


def to_dev(x: np.ndarray, device="cuda:0") -> torch.Tensor:
    """uint16 arrays are bf16 bit patterns; everything else keeps its dtype."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    return float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))


TOL = {"f32": 1e-5, "bf16": 2e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
