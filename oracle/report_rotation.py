"""Report: attention error of K4V2 with and without key rotation, against K4V4.

TEST INFRASTRUCTURE ONLY: a measurement script over the oracle and the seeded input
generators; the HIP library never calls it.

"Quantize What Counts" (technical summary: contributions, orthogonality and
integration; results, rotation integration) reports that rotating only the keys
before quantization brings K4V2 close to K4V4.  This script measures that claim on
the synthetic workloads: for every (seed, batch row, KV head) slab it packs the keys
and values with the library's format (keys per channel over 32-token groups,
values per token over 32-channel groups; every token quantized, no fp16 window, so
the quantizer alone decides the error), decodes the slab's query heads and compares
with exact float64 attention over the unquantized keys and values.  Per slab it
takes the max and the mean of |out - exact| over the heads and channels; the table
gives the mean and the max of those over all slabs.

It also reports the reconstruction error of keys and of values at equal bits (2 and
4), relative (||x_hat - x|| / ||x||) and absolute (RMS of x_hat - x), the comparison
behind "keys get more bits" ("Quantize What Counts", results: reconstruction error;
methodology: keys take more bits than values).

A second block quantizes keys per token instead (groups of 32 adjacent channels of
one token, the quantizer layout the pages' backends apply to keys), so that the
effect of the rotation can be read for both key layouts.

    python -m oracle.report_rotation [--seeds N] [--T T]      (8 seeds: 32 slabs)
"""

import argparse

import numpy as np

from workloads import Workload, make_queries
from workloads.synth import make_slab

from .kvq_oracle import (attention, decode_slab, default_scale, dequant_slab, hadamard_rotate, pack_slab,
                         quantize_groups, rotate_query, upcast)


def per_token_keys(K32: np.ndarray, bits: int) -> np.ndarray:
    """Keys quantized per token in groups of 32 adjacent channels, dequantized
    (code * s + z in float64)."""
    T, Dk = K32.shape
    c, s, z = quantize_groups(K32.reshape(T, Dk // 32, 32), bits)
    return (c.astype(np.float64) * s.astype(np.float64)[..., None] + z.astype(np.float64)[..., None]).reshape(T, Dk)


def value_hat(V32: np.ndarray, bits: int) -> np.ndarray:
    T, Dv = V32.shape
    c, s, z = quantize_groups(V32.reshape(T, Dv // 32, 32), bits)
    return (c.astype(np.float64) * s.astype(np.float64)[..., None] + z.astype(np.float64)[..., None]).reshape(T, Dv)


def recon_errors(w: Workload, b: int, h: int):
    """{bits: (K relative, V relative, K RMS, V RMS)} of one slab, library format."""
    sl = make_slab(w, b, h, 0, w.T)
    K32, V32 = upcast(sl.K, w.dtype).astype(np.float64), upcast(sl.V, w.dtype).astype(np.float64)
    out = {}
    for bits in (2, 4):
        p = pack_slab(sl.K, sl.V, w.dtype, bits, bits, 0, 0)
        Kh, Vh = dequant_slab(p, bits, bits)
        out[bits] = (np.linalg.norm(Kh - K32) / np.linalg.norm(K32), np.linalg.norm(Vh - V32) / np.linalg.norm(V32),
                     np.sqrt(np.mean((Kh - K32) ** 2)), np.sqrt(np.mean((Vh - V32) ** 2)))
    return out


def slab_errors(w: Workload, b: int, h: int, q_all):
    """{label: (max |err|, mean |err|)} of one slab."""
    sl = make_slab(w, b, h, 0, w.T)
    G = w.Hq // w.Hkv
    q = q_all[b, h * G:(h + 1) * G]
    scale = default_scale(w.Dk)
    K32, V32, q32 = upcast(sl.K, w.dtype), upcast(sl.V, w.dtype), upcast(q, w.dtype)
    exact = attention(q32, K32, V32, scale)
    out = {}
    for kb, vb, rot in [(4, 4, False), (4, 2, False), (4, 2, True), (2, 4, False), (2, 4, True), (2, 2, False),
                        (2, 2, True)]:
        p = pack_slab(sl.K, sl.V, w.dtype, kb, vb, 0, 0, key_rotation=rot)
        o = decode_slab(q, p, w.dtype, kb, vb, scale, key_rotation=rot)
        e = np.abs(o - exact)
        out["per-channel K%dV%d%s" % (kb, vb, " rot" if rot else "")] = (e.max(), e.mean())
    for kb, vb, rot in [(4, 4, False), (4, 2, False), (4, 2, True), (2, 4, False), (2, 4, True)]:
        Kx = hadamard_rotate(K32) if rot else K32
        Khat = per_token_keys(Kx, kb)
        qq = rotate_query(q32) if rot else q32
        o = attention(qq, Khat, value_hat(V32, vb), scale)
        e = np.abs(o - exact)
        out["per-token   K%dV%d%s" % (kb, vb, " rot" if rot else "")] = (e.max(), e.mean())
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seeds", type=int, default=8)
    ap.add_argument("--T", type=int, default=2048)
    args = ap.parse_args()
    rows = {}
    recon = {2: [], 4: []}
    n = 0
    for seed in range(args.seeds):
        w = Workload("rotation_report", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=args.T, k_bits=4, v_bits=2,
                     dtype="bf16", seed=100 + seed)
        q_all = make_queries(w)
        for b in range(w.B):
            for h in range(w.Hkv):
                for k, v in slab_errors(w, b, h, q_all).items():
                    rows.setdefault(k, []).append(v)
                for bits, v in recon_errors(w, b, h).items():
                    recon[bits].append(v)
                n += 1
    print("%d slabs (%d seeds x 2 batch rows x 2 KV heads), T = %d, Dk = Dv = 128, G = 4, bf16 inputs"
          % (n, args.seeds, args.T))
    print("%-22s %12s %12s %12s %12s" % ("keys", "mean max|e|", "max max|e|", "mean mean|e|", "max mean|e|"))
    for k, v in rows.items():
        a = np.array(v)
        print("%-22s %12.3e %12.3e %12.3e %12.3e" % (k, a[:, 0].mean(), a[:, 0].max(), a[:, 1].mean(), a[:, 1].max()))
    print("reconstruction error at equal bits (library format), mean [min, max] over slabs:")
    for bits, v in recon.items():
        a = np.array(v)
        print("  %d-bit  relative K %.3e [%.3e, %.3e]  V %.3e [%.3e, %.3e]   RMS K %.3e  V %.3e"
              % (bits, a[:, 0].mean(), a[:, 0].min(), a[:, 0].max(), a[:, 1].mean(), a[:, 1].min(), a[:, 1].max(),
                 a[:, 2].mean(), a[:, 3].mean()))


if __name__ == "__main__":
    main()
