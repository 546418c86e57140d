"""Host <-> device conversions shared by the GPU tests (no method arithmetic here)."""
import numpy as np
import torch

DEV = "cuda:0"


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 device tensor (same bits)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    b = bf16_bits(t)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
