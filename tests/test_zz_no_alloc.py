"""kv_decode_attn_noalloc: the decode without a workspace, its partial results in
the library's static per-GPU scratch.  Through the C ABI, each call must equal
kv_decode_attn with a caller workspace on the same inputs (same kernels, same
split: bit for bit) and the oracle within 2e-3; two calls in a row, the second on a
smaller input, then a call on the vector-ALU kernel, then one whose partial results
would not fit, which must be refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import MAX_ABS_ERR
from quantized_decode_attention_kv_amd import _lib as L_
from quantized_decode_attention_kv_amd import api
from workloads import Workload, make_all, make_queries
from workloads.device import to_device

pytestmark = pytest.mark.gpu

CASES = [
    # matrix-core kernel, 5 partitions cut into 40 units per slab
    Workload("noalloc_k4v2", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=1064, k_bits=4, v_bits=2, n_recent=40,
             dtype="bf16", partitions=5, seed=51),
    # a smaller input on the same scratch
    Workload("noalloc_small", B=1, Hq=4, Hkv=1, Dk=64, Dv=128, T=332, k_bits=4, v_bits=4, n_recent=12,
             dtype="f16", partitions=3, seed=52),
    # vector-ALU kernel (2 query heads per KV head)
    Workload("noalloc_valu", B=1, Hq=4, Hkv=2, Dk=64, Dv=96, T=579, k_bits=2, v_bits=4, log_window=32,
             dtype="f32", partitions=4, seed=53),
]


def _run(w):
    print("noalloc case %s P=%d" % (w.name, w.partitions), flush=True)
    K, V = make_all(w, workers=4)
    q = make_queries(w)
    lay = api.Layout.from_workload(w)
    cache = api.kv_quant_pack(lay, to_device(K, w.dtype), to_device(V, w.dtype))
    qd = to_device(q, w.dtype)
    scale = float(O.default_scale(w.Dk))
    ref = api.kv_decode_attn(lay, qd, cache, num_partitions=w.partitions, softmax_scale=scale)
    out = torch.full_like(ref, float("nan"))
    api.kv_decode_attn_noalloc(lay, qd, cache, num_partitions=w.partitions, softmax_scale=scale, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), (w.name, (out - ref).abs().max().item())
    want = O.decode_all(q, O.pack_all(K, V, w), w, scale)
    err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
    print("  equal to kv_decode_attn; max|err| vs oracle %.2e" % err, flush=True)
    assert err <= MAX_ABS_ERR, (w.name, err)


def test_noalloc_matches_workspace_decode_twice_then_smaller():
    for w in CASES:
        _run(w)


def test_noalloc_refuses_partials_beyond_the_scratch():
    # 32 x 32 query heads x 64 partitions x 132 floats = 34.6 MB of partial rows
    lay = api.Layout(32, 32, 8, 128, 128, 32768, 4, 2, 128, 0)
    assert lay.workspace_bytes(64) > L_.KVQ_STATIC_SCRATCH_BYTES
    fake = 1 << 20   # never dereferenced: the call is refused before any launch
    c = L_.KvqCache(*([fake] * 8))
    st = L_.load().kv_decode_attn_noalloc(lay.ref, ctypes.c_void_p(fake), L_.KVQ_BF16, ctypes.byref(c),
                                          ctypes.c_float(0.1), 64, ctypes.c_void_p(fake), None)
    assert st == L_.KVQ_ERR_UNSUPPORTED
    assert b"static scratch" in L_.load().kvq_last_error()
