"""Moving generated workload arrays to a torch device (data plumbing only)."""
import numpy as np
import torch


def to_dev(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage-typed numpy array (float32, or uint16 bf16 bits) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to(device)


def norm_torch_dtype(norm_dtype: str):
    return torch.float16 if norm_dtype == "f16" else torch.float32


def norms_to_dev(vn64: np.ndarray, norm_dtype: str, device) -> torch.Tensor:
    """Float64 values of stored value norms -> device tensor of the storage type."""
    if norm_dtype == "f16":
        return torch.from_numpy(vn64.astype(np.float16)).to(device)
    return torch.from_numpy(vn64.astype(np.float32)).to(device)
