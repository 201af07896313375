"""Helpers for the GPU tests: move seeded numpy inputs to the device."""
import numpy as np
import torch


def bf16(bits: np.ndarray, dev) -> torch.Tensor:
    """uint16 bf16 storage bits -> torch.bfloat16 on `dev` (same bits)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)


def f32(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def i32(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits32(t: torch.Tensor) -> np.ndarray:
    return host(t).view(np.uint32)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def say(msg: str):
    print(msg, flush=True)
