"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device and
packed buffers back.  No arithmetic of the method lives here."""

import numpy as np
import torch

from workloads.device import to_device, upload_workload  # noqa: F401

MAX_ABS_ERR = 2e-3   # decode output bound against the oracle's float64 attention


def cache_to_numpy(cache) -> dict:
    """Device cache tensors -> numpy arrays with the oracle's dtypes (uint32 codes, uint16 fp16 bits)."""
    out = {}
    for k, t in cache.items():
        a = t.cpu().numpy()
        out[k] = {np.dtype(np.int32): np.uint32, np.dtype(np.float16): np.uint16}.get(a.dtype, None)
        out[k] = a.view(out[k]) if out[k] is not None else a
    return out


def cache_from_numpy(packed: dict, device="cuda") -> dict:
    """Oracle packed arrays -> device tensors of the library's cache dtypes."""
    out = {}
    for k, a in packed.items():
        if a.dtype == np.uint32:
            out[k] = torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)
        elif a.dtype == np.uint8:
            out[k] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(device)
    return out
