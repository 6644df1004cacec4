"""Host -> device plumbing for stored tensors (no arithmetic)."""
import numpy as np
import torch


def torch_dtype(storage):
    return torch.bfloat16 if storage == "bf16" else torch.float32


def to_device(arr, storage=None, device="cuda"):
    """numpy array -> contiguous device tensor.  bfloat16 data travels as its
    uint16 bit patterns and is reinterpreted, not converted."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a).to(device)
    return t.contiguous()
