"""Helpers for the GPU parity tests: host<->device transfer of bf16 bit
patterns and the error metrics the parity bars are stated in."""
import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy array -> CUDA tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """CUDA tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.numpy()


def combine_rel_err(y: np.ndarray, y_ref: np.ndarray) -> float:
    """max over tokens of max_d |y - y_ref| / max_d |y_ref| (the combine bar)."""
    if y.size == 0:
        return 0.0
    num = np.abs(y.astype(np.float64) - y_ref).max(axis=1)
    den = np.abs(y_ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def rel_l2(x: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(x.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
