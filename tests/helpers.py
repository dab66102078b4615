"""Shared test helpers: tensor <-> float64 numpy, error metrics, ulp distance."""
import numpy as np
import torch


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (CPU or GPU) bf16/fp32 tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def relF(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    ny = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / (ny if ny > 0 else 1.0))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().astype(np.int32)


def f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int32).numpy().astype(np.int64)


def ulp_distance(a: torch.Tensor, b: torch.Tensor) -> np.ndarray:
    """Distance in units in the last place between two same-dtype tensors
    (sign-magnitude bit patterns mapped onto a monotone integer line)."""
    if a.dtype == torch.bfloat16:
        ia, ib = bf16_bits(a), bf16_bits(b)
        sign = 1 << 15
    else:
        ia, ib = f32_bits(a), f32_bits(b)
        sign = 1 << 31

    def mono(i):
        i = i.astype(np.int64) & ((sign << 1) - 1)
        return np.where(i & sign, -(i & (sign - 1)), i)
    return np.abs(mono(ia) - mono(ib))
