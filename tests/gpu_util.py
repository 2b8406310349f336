"""Host <-> device plumbing for the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

DEV = "cuda"


def to_dev(a: np.ndarray, fmt: str = None) -> torch.Tensor:
    """NumPy array -> device tensor; fmt 'bf16' means `a` holds uint16 bf16 bits."""
    a = np.ascontiguousarray(a)
    if fmt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device output of any float dtype."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
