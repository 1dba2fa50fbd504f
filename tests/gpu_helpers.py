"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device and
packed buffers back.  No arithmetic of the method lives here."""

import numpy as np
import torch

from workloads import make_all, make_queries

MAX_ABS_ERR = 2e-3   # decode output bound against the oracle's float64 attention


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage-dtype numpy array -> torch tensor on the GPU (bf16 travels as bit patterns)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    raise ValueError(dtype)


def cache_to_numpy(cache) -> dict:
    """Device cache tensors -> numpy arrays with the oracle's dtypes (uint32 codes, uint16 fp16 bits)."""
    out = {}
    for k, t in cache.items():
        a = t.cpu().numpy()
        out[k] = a.view(np.uint32) if a.dtype == np.int32 else a.view(np.uint16)
    return out


def cache_from_numpy(packed: dict, device="cuda") -> dict:
    """Oracle packed arrays -> device tensors of the library's cache dtypes."""
    out = {}
    for k, a in packed.items():
        if a.dtype == np.uint32:
            out[k] = torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(a).view(np.float16)).to(device)
    return out


def upload_workload(w, t_lo=0, t_hi=None, device="cuda"):
    """Draw every slab of K/V positions [t_lo, t_hi) and upload slab by slab (bounded
    host memory), plus the queries.  Returns (K, V, q) device tensors."""
    if t_hi is None:
        t_hi = w.T
    n = t_hi - t_lo
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    K = torch.empty((w.B, w.Hkv, n, w.Dk), dtype=tdt, device=device)
    V = torch.empty((w.B, w.Hkv, n, w.Dv), dtype=tdt, device=device)

    def sink(b, h, s):
        K[b, h].copy_(to_device(s.K, w.dtype, "cpu"))
        V[b, h].copy_(to_device(s.V, w.dtype, "cpu"))

    make_all(w, t_lo, t_hi, sink=sink)
    torch.cuda.synchronize()
    q = to_device(make_queries(w), w.dtype, device)
    return K, V, q
