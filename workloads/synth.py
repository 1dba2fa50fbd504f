"""Seeded synthetic KV caches and decode queries.

Value recipe (a stand-in for the activations of the trained models the pages evaluate
on, which are not available here):

* keys:   K[b,h,t,c] = z * m_c + mu[h,c],  z ~ N(0, 1),
          m_c = 8 on 4 distinct "outlier" channels per KV head, 1 elsewhere,
          mu[h,c] ~ N(0, std 2) per KV head and channel (a per-channel offset that is
          the same for every token and every batch row);
* values: V[b,h,t,c] ~ N(0, std 0.5);
* query:  q[b,i,c] ~ N(0, 1).

Streams are independent per unit so any slab can be drawn alone:
``SeedSequence([seed, 1, h])`` draws the per-head outlier channels and offsets,
``SeedSequence([seed, 2, b, h])`` draws the (T, Dk) keys then the (T, Dv) values of
slab (b, h), ``SeedSequence([seed, 3, b])`` draws the (Hq, Dk) queries of row b.
All draws are float32; for bf16 (fp16) workloads the float32 values are rounded to
the nearest bf16 (fp16), ties to even, and handed over as uint16 bit patterns.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

from .configs import Workload


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _gen(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def head_params(w: Workload, h: int):
    """(channel multipliers m[Dk], offsets mu[Dk]) for KV head h, float32."""
    rng = _gen(w.seed, 1, h)
    n_out = min(w.n_outliers, w.Dk)
    outliers = rng.choice(w.Dk, size=n_out, replace=False)
    mu = rng.standard_normal(w.Dk, dtype=np.float32) * np.float32(w.k_offset_std)
    m = np.ones(w.Dk, dtype=np.float32)
    m[outliers] = np.float32(w.outlier_scale)
    return m, mu


@dataclass
class SlabInputs:
    """K [T, Dk] and V [T, Dv] of one (b, h) slab in the workload's storage dtype
    (float32, or uint16 bf16 bit patterns)."""
    K: np.ndarray
    V: np.ndarray


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32, copy=False)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)   # numpy rounds to nearest, ties to even
    raise ValueError(dtype)


def make_slab(w: Workload, b: int, h: int, t_lo: int = 0, t_hi: int = None) -> SlabInputs:
    """Keys and values of slab (b, h), positions [t_lo, t_hi) (the whole stream is drawn
    so that a sub-range equals the same rows of the full slab)."""
    if t_hi is None:
        t_hi = w.T
    m, mu = head_params(w, h)
    rng = _gen(w.seed, 2, b, h)
    z = rng.standard_normal((w.T, w.Dk), dtype=np.float32)
    K = z[t_lo:t_hi] * m + mu
    del z
    V = rng.standard_normal((w.T, w.Dv), dtype=np.float32)[t_lo:t_hi] * np.float32(w.v_std)
    return SlabInputs(_to_storage(K, w.dtype), _to_storage(V, w.dtype))


def make_queries(w: Workload) -> np.ndarray:
    """q [B, Hq, Dk] in storage dtype."""
    q = np.stack([_gen(w.seed, 3, b).standard_normal((w.Hq, w.Dk), dtype=np.float32)
                  for b in range(w.B)])
    return _to_storage(q, w.dtype)


def make_all(w: Workload, t_lo: int = 0, t_hi: int = None, workers: int = None,
             sink=None):
    """Draw every slab.  Returns (K [B,Hkv,t,Dk], V [B,Hkv,t,Dv]) numpy arrays in
    storage dtype, or, if ``sink(b, h, slab)`` is given, hands each slab to it instead
    (so a caller can upload slab by slab without holding the whole cache on the host)."""
    if t_hi is None:
        t_hi = w.T
    n = t_hi - t_lo
    sdt = np.float32 if w.dtype == "f32" else np.uint16
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    K = V = None
    if sink is None:
        K = np.empty((w.B, w.Hkv, n, w.Dk), dtype=sdt)
        V = np.empty((w.B, w.Hkv, n, w.Dv), dtype=sdt)

    def one(bh):
        b, h = bh
        s = make_slab(w, b, h, t_lo, t_hi)
        if sink is None:
            K[b, h] = s.K
            V[b, h] = s.V
        else:
            sink(b, h, s)

    units = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    if workers == 1 or len(units) == 1:
        for u in units:
            one(u)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, units))
    return K, V
