"""kv_decode_attn captured in a HIP graph (through torch.cuda.graph) and replayed.

The library enqueues only on the caller's stream and records no memset, so a decode
(decode kernel + merge) can be captured once and replayed.  Every replay is checked
against the eager result of the same call, with eager work and synchronizations
between the replays; the query is changed in place between replays, as a serving
loop would, and the expected output is recomputed eagerly each time.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import MAX_ABS_ERR
from quantized_decode_attention_kv_amd import api
from workloads import make_queries, small_cases
from workloads.device import to_device, upload_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [0, 1])
def test_decode_graph_replays(idx):
    w = small_cases()[idx]
    print("graph case %s" % w.name, flush=True)
    lay = api.Layout.from_workload(w)
    Kd, Vd, qd = upload_workload(w)
    cache = api.kv_quant_pack(lay, Kd, Vd)
    P = w.partitions
    scale = float(O.default_scale(w.Dk))
    ws = api.alloc_workspace(lay, P)
    out_g = torch.empty((w.B, w.Hq, w.Dv), dtype=torch.float32, device="cuda")
    q_g = qd.clone()
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        api.kv_decode_attn(lay, q_g, cache, num_partitions=P, softmax_scale=scale, out=out_g, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.kv_decode_attn(lay, q_g, cache, num_partitions=P, softmax_scale=scale, out=out_g, workspace=ws)
    torch.cuda.synchronize()

    rng = np.random.default_rng(61)
    ws_e = api.alloc_workspace(lay, P)
    for rep in range(3):
        q_new = to_device(make_queries(w.with_(seed=w.seed + 100 + rep)), w.dtype)
        q_g.copy_(q_new)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = api.kv_decode_attn(lay, q_new, cache, num_partitions=P, softmax_scale=scale, workspace=ws_e)
        _ = torch.randn(int(rng.integers(1000, 5000)), device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        err = (out_g - want).abs().max().item()
        assert err <= 1e-6, (w.name, rep, err)   # same kernels, same inputs: the same result
        # and within the oracle's tolerance
        if rep == 0:
            ref = O.decode_all(make_queries(w.with_(seed=w.seed + 100)), O.pack_all(*_host_inputs(w), w), w, scale)
            assert np.abs(out_g.cpu().numpy().astype(np.float64) - ref).max() <= MAX_ABS_ERR


def _host_inputs(w):
    from workloads import make_all
    return make_all(w, workers=4)
