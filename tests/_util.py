"""Helpers shared by the tests (no step of the method lives here)."""
import numpy as np


def to_torch(arr, dtype: str, device="cuda"):
    """Host array in the generator's stored form -> torch tensor of that dtype on device."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def upper_to_full(Hu: np.ndarray) -> np.ndarray:
    """Symmetric matrix from its upper triangle."""
    return np.triu(Hu) + np.triu(Hu, 1).T


def compare_codes(got: np.ndarray, ref: np.ndarray):
    """(fraction identical, max |difference|)."""
    got = got.astype(np.int64)
    ref = ref.astype(np.int64)
    same = float(np.mean(got == ref))
    mx = int(np.abs(got - ref).max()) if got.size else 0
    return same, mx
