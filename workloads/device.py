"""Moving seeded inputs to the GPU with torch (data movement only)."""

import numpy as np

from .synth import make_all, make_queries


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    """Storage-dtype numpy array -> torch tensor (bf16 and fp16 travel as bit patterns)."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.float16)
    raise ValueError(dtype)


def upload_workload(w, t_lo=0, t_hi=None, device="cuda"):
    """Draw every slab of K/V positions [t_lo, t_hi) and upload slab by slab (bounded
    host memory), plus the queries.  Returns (K, V, q) device tensors."""
    import torch
    if t_hi is None:
        t_hi = w.T
    n = t_hi - t_lo
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    K = torch.empty((w.B, w.Hkv, n, w.Dk), dtype=tdt, device=device)
    V = torch.empty((w.B, w.Hkv, n, w.Dv), dtype=tdt, device=device)

    def sink(b, h, s):
        K[b, h].copy_(to_device(s.K, w.dtype, "cpu"))
        V[b, h].copy_(to_device(s.V, w.dtype, "cpu"))

    make_all(w, t_lo, t_hi, sink=sink)
    torch.cuda.synchronize()
    q = to_device(make_queries(w), w.dtype, device)
    return K, V, q
