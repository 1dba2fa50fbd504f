"""HeadQ side code on the GPU ("HeadQ", section 3) against the oracle.

The write path (kv_side_pack) must match the oracle's side codes, scales and zeros
bit for bit.  Both sides sum the residual projection in float64 in channel order
and round it once to float32, so the quantizer sees the same values.  The read path
(kv_decode_attn_side) must match the oracle's corrected decode within 2e-3.  The
basis is orthonormal, from a seeded QR: the page's basis comes from calibration
queries, which do not exist here.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import MAX_ABS_ERR
from quantized_decode_attention_kv_amd import api
from workloads import make_all, make_queries, small_cases
from workloads.device import upload_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx,rank,bits", [(0, 4, 8), (3, 8, 4), (13, 16, 2), (19, 6, 4)])
def test_side_code_and_corrected_decode(idx, rank, bits):
    w = small_cases()[idx]
    print("headq case %s rank %d bits %d" % (w.name, rank, bits), flush=True)
    lay = api.Layout.from_workload(w)
    Kd, Vd, qd = upload_workload(w)
    cache = api.kv_quant_pack(lay, Kd, Vd)
    rng = np.random.default_rng(100 + idx)
    U = np.stack([np.linalg.qr(rng.standard_normal((w.Dk, rank)))[0] for _ in range(w.Hkv)]).astype(np.float32)
    Ud = torch.from_numpy(U).cuda()
    side = api.side_pack(lay, Kd, cache, Ud, side_bits=bits)
    out = api.kv_decode_attn_side(lay, qd, cache, Ud, side, num_partitions=w.partitions).cpu().numpy()
    torch.cuda.synchronize()
    codes, sc, zr = (t.cpu().numpy() for t in side)
    K, V = make_all(w, workers=4)
    q = make_queries(w)
    packed = O.pack_all(K, V, w)
    scale = float(O.default_scale(w.Dk))
    G = w.Hq // w.Hkv
    for b in range(w.B):
        for h in range(w.Hkv):
            p = O.slab_of(packed, b, h)
            want = O.headq_side_slab(K[b, h], w.dtype, p, U[h], w.k_bits, w.v_bits, w.n_recent, w.log_window, bits)
            assert np.array_equal(codes[b, h], want["side_codes"]), (b, h)
            assert np.array_equal(sc[b, h].view(np.uint16), want["side_scale"]), (b, h)
            assert np.array_equal(zr[b, h].view(np.uint16), want["side_zero"]), (b, h)
            ref = O.decode_slab_headq(q[b, h * G:(h + 1) * G], p, want, U[h], w.dtype, w.k_bits, w.v_bits, scale)
            err = np.abs(out[b, h * G:(h + 1) * G] - ref).max()
            assert err <= MAX_ABS_ERR, (b, h, err)
