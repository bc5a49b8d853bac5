"""Small test utilities (no attention arithmetic)."""
import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a tensor as numpy uint16 (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def err_stats(got, ref):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
