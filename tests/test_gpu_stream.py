"""GPU parity of the streaming cache (kv_stream_prefill / kv_stream_append /
kv_stream_decode) against the oracle's ``SlabStream``, through the C ABI.

After every checked step:
* every packed group (codes, fp16 scale / zero bits) equals the oracle's group of
  the same index bit for bit;
* every fp16 row in use equals the oracle's fp16 copy of the position the host
  state says it holds (rows may sit in any order; the position map is the unique
  part);
* decode is within 2e-3 (max abs) of the oracle's float64 attention over the same
  tokens, for several partition counts.
Small shapes check every slab; the two long-context shapes check sampled slabs.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle.kvq_stream import SlabStream
from gpu_helpers import MAX_ABS_ERR, cache_to_numpy
from quantized_decode_attention_kv_amd import api
from workloads import Workload, make_queries, workload
from workloads.device import upload_workload
from workloads.synth import make_slab

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _valid_prefill(w, near):
    """Largest T0 <= near whose quantized count is a multiple of 32."""
    for T0 in range(near, 0, -1):
        r, u = O.split_positions(T0, w.n_recent, w.log_window)
        if len(u) % 32 == 0:
            return T0
    raise AssertionError("no valid prefill length")


def _compare_slab(s, gpu, b, h, o: SlabStream, first_group=0, where=""):
    p, _, rpos = o.as_packed()
    nG = s.n_groups
    assert nG == len(o.groups), (where, nG, len(o.groups))
    g0 = first_group
    checks = {
        "k_codes": (gpu["k_codes"][b, h, 32 * g0:32 * nG], p["k_codes"][32 * g0:]),
        "k_scale": (gpu["k_scale"][b, h, g0:nG], p["k_scale"][g0:]),
        "k_zero": (gpu["k_zero"][b, h, g0:nG], p["k_zero"][g0:]),
        "v_codes": (gpu["v_codes"][b, h, g0:nG], p["v_codes"][g0:]),
        "v_scale": (gpu["v_scale"][b, h, g0:nG], p["v_scale"][g0:]),
        "v_zero": (gpu["v_zero"][b, h, g0:nG], p["v_zero"][g0:]),
    }
    for k, (g, r) in checks.items():
        assert g.shape == r.shape, (where, k, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError("%s slab (%d, %d) %s: %d mismatches, first at %s" % (where, b, h, k, len(bad), bad[0]))
    pos = s.row_positions()
    assert sorted(pos) == sorted(int(x) for x in rpos), where
    for i, t in enumerate(pos):
        kr, vr = o.rows[t]
        assert np.array_equal(gpu["k_fp16"][b, h, i], kr), (where, b, h, "k row", i, t)
        assert np.array_equal(gpu["v_fp16"][b, h, i], vr), (where, b, h, "v row", i, t)


def _check_decode(s, w, qd, q, oracles, slabs, partitions, where=""):
    scale = float(O.default_scale(w.Dk))
    G = w.Hq // w.Hkv
    max_p = max(1, (s.t + 31) // 32)
    want = {(b, h): oracles[(b, h)].decode(q[b, h * G:(h + 1) * G], w.dtype, scale) for (b, h) in slabs}
    for P in sorted({min(P, max_p) for P in partitions}):
        out = s.decode(qd, num_partitions=P, softmax_scale=scale)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        for (b, h) in slabs:
            err = np.abs(got[b, h * G:(h + 1) * G] - want[(b, h)]).max()
            assert err <= MAX_ABS_ERR, (where, P, b, h, err)


def _run_stream(w: Workload, T0: int, T1: int, check_at, partitions, slabs=None, group_window=None):
    """Prefill T0 tokens (0: start empty), append up to T1, compare at the steps in check_at."""
    _log("stream case %s T0=%d T1=%d" % (w.name, T0, T1))
    if slabs is None:
        slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    Kd, Vd, qd = upload_workload(w, 0, T1)
    q = make_queries(w)
    host = {}
    for (b, h) in slabs:
        sl = make_slab(w, b, h, 0, T1)
        host[(b, h)] = (sl.K, sl.V)
    s = api.Stream(w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T, w.k_bits, w.v_bits, w.n_recent, w.log_window,
                   v_group=w.v_group, key_rotation=w.key_rotation)
    oracles = {bh: SlabStream(w.Dk, w.Dv, w.k_bits, w.v_bits, w.n_recent, w.log_window, w.v_group,
                              key_rotation=w.key_rotation) for bh in slabs}
    if T0:
        s.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
        for bh, o in oracles.items():
            o.prefill(host[bh][0][:T0], host[bh][1][:T0], w.dtype)
    for t in range(T0, T1):
        s.append(Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous())
        for bh, o in oracles.items():
            o.append(host[bh][0][t], host[bh][1][t], w.dtype)
        if s.t in check_at or s.t == T1:
            torch.cuda.synchronize()
            gpu = cache_to_numpy(s.cache)
            first = 0 if group_window is None else max(0, s.n_groups - group_window)
            for (b, h), o in oracles.items():
                _compare_slab(s, gpu, b, h, o, first, "%s t=%d" % (w.name, s.t))
            _check_decode(s, w, qd, q, oracles, slabs, partitions, "%s t=%d" % (w.name, s.t))
    _log("  ok: %d groups, %d fp16 rows, %d pending" % (s.n_groups, s.n_rows, s.n_pending))
    return s


def test_stream_window_from_empty():
    """K4V2, 40-token fp16 window, no log spacing, from an empty stream."""
    w = Workload("stream_k4v2_win", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=400, k_bits=4, v_bits=2,
                 n_recent=40, dtype="bf16", seed=21)
    _run_stream(w, 0, 330, {1, 2, 40, 41, 72, 73, 105, 200}, [1, 3])


def test_stream_log_window_after_prefill():
    """K2V2 with log-spaced fp16 tokens (window 64), after a one-shot prefill."""
    w = Workload("stream_k2v2_log", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=2600, k_bits=2, v_bits=2,
                 n_recent=64, log_window=64, dtype="bf16", seed=22)
    T0 = _valid_prefill(w, 2000)
    _run_stream(w, T0, T0 + 420, {T0 + 1, T0 + 64, T0 + 200, T0 + 333}, [1, 7])


def test_stream_every_token_pending_f32():
    """No fp16 window: each token is pending at once and every 32nd append packs a
    group that contains the token being appended (thin keys, K8V4, float32 inputs
    rounded to fp16 first)."""
    w = Workload("stream_k8v4_thin", B=2, Hq=8, Hkv=2, Dk=32, Dv=128, T=300, k_bits=8, v_bits=4,
                 dtype="f32", seed=23)
    _run_stream(w, 0, 260, {1, 31, 32, 33, 64, 96, 128}, [1, 4])


def test_stream_g8_odd_widths():
    """G = 8, Dk = 96, Dv = 64, K2V4, window 32 with log spacing 32 (generic kernel)."""
    w = Workload("stream_g8_k2v4", B=1, Hq=16, Hkv=2, Dk=96, Dv=64, T=1500, k_bits=2, v_bits=4,
                 n_recent=32, log_window=32, dtype="bf16", seed=24)
    _run_stream(w, 0, 1100, {100, 257, 513, 800}, [1, 2, 5])


def test_stream_value_groups_128():
    """Values in groups of 128 channels (one scale per token row): the append
    kernel's group minima and maxima span two waves."""
    w = Workload("stream_k4v2_vg128", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=300, k_bits=4, v_bits=2,
                 n_recent=16, dtype="bf16", seed=26, v_group=128)
    _run_stream(w, 0, 240, {17, 48, 49, 112, 200}, [1, 3])


def test_stream_value_groups_64_generic():
    """Values in groups of 64 channels with 64-wide heads and G = 2 (generic decode
    kernel), float32 inputs, after a prefill."""
    w = Workload("stream_g2_vg64", B=1, Hq=4, Hkv=2, Dk=64, Dv=64, T=500, k_bits=8, v_bits=4,
                 n_recent=32, log_window=16, dtype="f32", seed=27, v_group=64)
    T0 = _valid_prefill(w, 200)
    _run_stream(w, T0, T0 + 200, {T0 + 1, T0 + 77, T0 + 150}, [1, 2])


def test_stream_f16_inputs_log_after_prefill():
    """fp16 keys, values and queries (K4V2, log-spaced fp16 tokens), after a prefill."""
    w = Workload("stream_k4v2_f16_log", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1400, k_bits=4, v_bits=2,
                 n_recent=64, log_window=64, dtype="f16", seed=31)
    T0 = _valid_prefill(w, 900)
    _run_stream(w, T0, T0 + 200, {T0 + 1, T0 + 64, T0 + 199}, [1, 3])


def test_stream_one_bit():
    """1-bit keys and values in a stream (the append kernel's 1-bit words), f32 inputs."""
    w = Workload("stream_k1v1", B=1, Hq=4, Hkv=2, Dk=64, Dv=128, T=300, k_bits=1, v_bits=1,
                 n_recent=8, dtype="f32", seed=28)
    _run_stream(w, 0, 200, {9, 40, 41, 104, 160}, [1, 2])


def test_stream_three_bit():
    """3-bit keys and values in a stream (bit streams with straddling codes; Dk = 96
    gives 9-word key rows)."""
    w = Workload("stream_k3v3", B=1, Hq=4, Hkv=2, Dk=96, Dv=128, T=300, k_bits=3, v_bits=3,
                 n_recent=8, dtype="bf16", seed=29)
    _run_stream(w, 0, 200, {9, 40, 41, 104, 160}, [1, 2])


def test_stream_three_bit_values_log_after_prefill():
    """K2V3 with 64-channel value groups and log-spaced fp16 tokens, after a prefill."""
    w = Workload("stream_k2v3_log_vg64", B=1, Hq=8, Hkv=2, Dk=128, Dv=128, T=1400, k_bits=2, v_bits=3,
                 n_recent=64, log_window=64, dtype="f32", seed=30, v_group=64)
    T0 = _valid_prefill(w, 900)
    _run_stream(w, T0, T0 + 300, {T0 + 1, T0 + 64, T0 + 299}, [1, 3])


def test_stream_key_rotation_after_prefill():
    """Rotated keys in a stream: K4V2 with log-spaced fp16 tokens after a prefill (the
    pack kernel's rotated groups and rows), then appends that rotate each new key row
    before its fp16 copy and form groups from rotated rows (MFMA decode, rotated q)."""
    w = Workload("stream_k4v2_rot", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1400, k_bits=4, v_bits=2,
                 n_recent=64, log_window=64, dtype="bf16", seed=32, key_rotation=True)
    T0 = _valid_prefill(w, 900)
    _run_stream(w, T0, T0 + 200, {T0 + 1, T0 + 64, T0 + 199}, [1, 3])


def test_stream_key_rotation_generic_from_empty():
    """Rotated 64-wide keys, G = 2 (vector-ALU decode), float32 inputs, K8V4, from an
    empty stream."""
    w = Workload("stream_g2_rot", B=1, Hq=4, Hkv=2, Dk=64, Dv=64, T=300, k_bits=8, v_bits=4,
                 n_recent=16, dtype="f32", seed=33, key_rotation=True)
    _run_stream(w, 0, 200, {17, 48, 49, 112}, [1, 2])


def test_stream_full_capacity_and_errors():
    """A stream filled to its capacity refuses another token and keeps its state."""
    w = Workload("stream_full", B=1, Hq=4, Hkv=1, Dk=64, Dv=64, T=96, k_bits=4, v_bits=4,
                 n_recent=16, dtype="bf16", seed=25)
    s = _run_stream(w, 0, 96, {96}, [1, 2])
    k = torch.zeros((1, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.L_.KvqError):
        s.append(k, k)
    assert s.t == 96
    with pytest.raises(api.L_.KvqError):
        s.prefill(torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16, device="cuda"))


def test_stream_long_128k_shape():
    """The 128K-token K4V2 shape (B4, 8 KV heads, D128, 128-token window): prefill to
    just under the full length, append 192 tokens (6 groups), sampled slabs."""
    w = workload("long_128k")
    T0 = _valid_prefill(w, w.T - 192)
    _run_stream(w, T0, T0 + 192, {T0 + 1, T0 + 32, T0 + 97}, [1, 64], slabs=[(0, 0), (3, 7)], group_window=8)


def test_stream_logquant_32k_shape():
    """The 32K-token K2V2 shape with log-spaced fp16 tokens (B32, 8 KV heads):
    prefill, then 160 appends, sampled slabs."""
    w = workload("logquant_32k")
    T0 = _valid_prefill(w, w.T - 160)
    _run_stream(w, T0, T0 + 160, {T0 + 1, T0 + 80}, [1, 16], slabs=[(0, 0), (31, 7)], group_window=8)
