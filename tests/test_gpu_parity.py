"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

* kv_quant_pack: codes and fp16 scale/zero bit patterns equal the oracle's bit for
  bit (the quantizer is a deterministic float32 recipe; nothing may differ).
* kv_decode_attn: float32 output within 2e-3 (max abs) of the oracle's float64
  attention over the same dequantized cache, fed first the oracle's packed cache,
  then the GPU's own.  Partition count and order are free (any split of the
  tokens gives the same attention), so several partition counts are checked.

Small shapes run whole; the five benchmark workloads run at full size, comparing
every packed byte where the oracle is fast enough and a sample of (batch, kv head)
slabs otherwise.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import MAX_ABS_ERR, cache_from_numpy, cache_to_numpy, to_device, upload_workload
from oracle_slabs import slab_references
from quantized_decode_attention_kv_amd import api
from workloads import WORKLOADS, Workload, make_all, make_queries, small_cases, workload

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _compare_pack(gpu: dict, ref: dict, where=""):
    for k in O.CACHE_KEYS:
        g, r = gpu[k], ref[k]
        assert g.shape == r.shape, (k, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError("%s%s: %d mismatches, first at %s: gpu %s oracle %s"
                                 % (where, k, len(bad), bad[0].tolist(), g[tuple(bad[0])], r[tuple(bad[0])]))


def _run_small(w: Workload, partitions=None, kernel=None):
    """Pack and decode the whole workload; returns (cache, oracle arrays, {P: plan}).
    kernel: the decode kernel every partition count must run on ("mfma" / "valu")."""
    _log("case %s (%s)" % (w.name, w.dtype))
    K, V = make_all(w, workers=4)
    q = make_queries(w)
    lay = api.Layout.from_workload(w)
    Kd, Vd, qd = to_device(K, w.dtype), to_device(V, w.dtype), to_device(q, w.dtype)
    cache = api.kv_quant_pack(lay, Kd, Vd)
    torch.cuda.synchronize()
    ref = O.pack_all(K, V, w)
    _compare_pack(cache_to_numpy(cache), ref, w.name + " ")
    scale = float(O.default_scale(w.Dk))
    want = O.decode_all(q, ref, w, scale)
    oracle_cache = cache_from_numpy(ref)
    max_p = max(1, (w.T + 31) // 32)
    plans = {}
    for P in partitions or sorted(p for p in {1, 2, w.partitions, max_p} if p <= max_p):
        plans[P] = plan = api.decode_plan(lay, P)
        if kernel is not None:
            assert plan["kernel"] == kernel, (w.name, P, plan)
        errs = []
        for name, c in (("oracle-packed", oracle_cache), ("gpu-packed", cache)):
            out = api.kv_decode_attn(lay, qd, c, num_partitions=P, softmax_scale=scale)
            torch.cuda.synchronize()
            err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
            errs.append(err)
            assert err <= MAX_ABS_ERR, (w.name, name, P, err)
        _log("  P=%d %s kernel, %d units, ring %d: max|err| %.2e (oracle-packed) %.2e (gpu-packed)"
             % (P, plan["kernel"], plan["units"], plan["ring_depth"], errs[0], errs[1]))
    return cache, ref, plans


def _expected_kernel(w: Workload) -> str:
    """The decode kernel include/kvq.h promises for a layout (no side code)."""
    mfma = (w.Hq == 4 * w.Hkv and w.Dv == 128 and w.Dk in (32, 64, 128) and w.k_bits in (2, 4, 8)
            and w.v_bits in (2, 4, 8) and w.Dk * w.k_bits >= 128)
    return "mfma" if mfma else "valu"


@pytest.mark.parametrize("w", small_cases(), ids=lambda w: w.name)
def test_small_cases(w):
    _run_small(w, kernel=_expected_kernel(w))


# Every (Dk, key bits, value bits) instance the matrix-core kernel is built for:
# Dk in {32, 64, 128}, 2/4/8-bit codes with at least 4 key-code bytes per lane.
MFMA_INSTANCES = [(dk, kb, vb) for dk in (32, 64, 128) for kb in (2, 4, 8) for vb in (2, 4, 8)
                  if dk * kb // 32 >= 4]
_DTYPES = ("bf16", "f16", "f32")


def test_mfma_instance_list():
    assert len(MFMA_INSTANCES) == 24


@pytest.mark.parametrize("dk,kb,vb", MFMA_INSTANCES, ids=lambda x: str(x))
def test_mfma_instances(dk, kb, vb):
    """Each matrix-core instance on a small cache: 2 batch rows x 2 KV heads, 10 code
    groups per slab plus a 12-token fp16 window, one, three and four partitions (the
    last cut into more units than there are groups); the input dtype cycles through
    bf16, fp16 and fp32 so every dtype meets the matrix-core kernel at several key widths."""
    i = MFMA_INSTANCES.index((dk, kb, vb))
    # 128-wide keys take 16-bit inputs only, so that every bit pair also runs through
    # the 16-bit inputs' dedicated pack kernel (fp32 meets the other key widths)
    dtype = _DTYPES[i % 2] if dk == 128 else _DTYPES[i % 3]
    w = Workload("mfma_d%d_k%dv%d" % (dk, kb, vb), B=2, Hq=8, Hkv=2, Dk=dk, Dv=128, T=332, k_bits=kb, v_bits=vb,
                 n_recent=12, dtype=dtype, partitions=4, seed=100 + i)
    _run_small(w, partitions=[1, 3, 4], kernel="mfma")


def test_tiny_ref_full():
    """The 256-token fp32 reference workload, whole."""
    _run_small(workload("tiny_ref"), kernel="valu")


def test_llama8b_gqa_4k_full():
    """Llama-8B-shaped GQA decode at 4096 tokens, every slab compared, at partition
    counts that take both of the matrix-core kernel's ring depths, 3 and 2 (128
    partitions put more waves on the device than the 3-deep ring fits, and give
    units without key groups)."""
    _, _, plans = _run_small(workload("llama8b_gqa_4k"), partitions=[1, 4, 16, 40, 128], kernel="mfma")
    assert {p["ring_depth"] for p in plans.values()} == {2, 3}, plans


def test_many_teams_one_slab():
    """One slab cut into many units: 64 and 256 partitions of 8 units give 128 and
    512 teams of four waves, at and past the 128 teams whose run starts the host
    passes with the launch (past it the kernel computes them itself), and most units
    hold one key group or none."""
    w = Workload("many_teams", B=1, Hq=4, Hkv=1, Dk=128, Dv=128, T=8224, k_bits=4, v_bits=2, n_recent=32,
                 dtype="bf16", partitions=256, seed=36)
    _, _, plans = _run_small(w, partitions=[64, 256], kernel="mfma")
    assert plans[64]["units"] == 512 and plans[256]["units"] == 2048, plans


def test_units_per_slab_four_and_not_a_multiple_of_four():
    """520 slabs with 2 or 3 partitions: the plan cuts each partition into 2 units,
    so with 2 partitions a slab is one team of four units whose combined state is the
    output itself (no merge), and with 3 partitions its 6 units are teams of their
    own that each write a partial row (unit counts not a multiple of 4)."""
    w = Workload("team_per_slab", B=130, Hq=16, Hkv=4, Dk=128, Dv=128, T=96, k_bits=4, v_bits=2, n_recent=32,
                 dtype="bf16", partitions=2, seed=38)
    _, _, plans = _run_small(w, partitions=[2, 3], kernel="mfma")
    assert plans[2]["units"] == 4 and plans[3]["units"] == 6, plans


@pytest.mark.parametrize("w", [
    Workload("one_group", B=1, Hq=4, Hkv=4, Dk=32, Dv=32, T=32, k_bits=2, v_bits=8, dtype="bf16", seed=31),
    Workload("all_fp16", B=2, Hq=8, Hkv=2, Dk=128, Dv=128, T=200, k_bits=4, v_bits=2, n_recent=200,
             dtype="bf16", partitions=3, seed=32),
    Workload("one_group_plus_fp16", B=1, Hq=2, Hkv=2, Dk=64, Dv=64, T=33, k_bits=4, v_bits=4, n_recent=1,
             dtype="f32", seed=33),
    Workload("max_dims_g16", B=1, Hq=16, Hkv=1, Dk=256, Dv=256, T=608, k_bits=8, v_bits=8, n_recent=32,
             dtype="bf16", partitions=5, seed=34),
    Workload("g1_wide_v", B=3, Hq=3, Hkv=3, Dk=32, Dv=256, T=256, k_bits=4, v_bits=2, dtype="bf16",
             partitions=8, seed=35),
], ids=lambda w: w.name)
def test_edge_cases(w):
    _run_small(w)


def test_pack_deterministic_and_chunked():
    """Two packs are bit-identical, and packing the cache in chunks that end on key
    group boundaries gives the same bytes as one pack (the prefill-append path)."""
    w = small_cases()[1]   # log-spaced retention: chunks cut through retained regions
    K, V = make_all(w, workers=4)
    lay = api.Layout.from_workload(w)
    Kd, Vd = to_device(K, w.dtype), to_device(V, w.dtype)
    a = cache_to_numpy(api.kv_quant_pack(lay, Kd, Vd))
    b = cache_to_numpy(api.kv_quant_pack(lay, Kd, Vd))
    _compare_pack(a, b, "repeat ")
    # cut points where the quantized count before the cut is a multiple of 32
    u = O.split_positions(w.T, w.n_recent, w.log_window)[1]
    cuts = [0] + [int(u[k]) for k in range(32 * 7, len(u), 32 * 13)] + [w.T]
    chunked = {k: torch.zeros_like(v) for k, v in api.alloc_cache(lay).items()}
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        api.kv_quant_pack(lay, Kd[:, :, t0:t1].contiguous(), Vd[:, :, t0:t1].contiguous(), cache=chunked, t_begin=t0)
    torch.cuda.synchronize()
    _compare_pack(cache_to_numpy(chunked), a, "chunked ")


def test_pack_rejects_group_splitting_chunk():
    w = small_cases()[0]
    lay = api.Layout.from_workload(w)
    K = torch.zeros((w.B, w.Hkv, 100, w.Dk), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros((w.B, w.Hkv, 100, w.Dv), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.L_.KvqError):
        api.kv_quant_pack(lay, K, V, cache=api.alloc_cache(lay), t_begin=0)


def test_constant_and_degenerate_groups():
    """Constant key channels and value rows quantize to all-zero codes with s = +0 and
    the dequantized value equal to fp16(x); signed zeros are stored as +0."""
    w = Workload("const", B=1, Hq=2, Hkv=1, Dk=64, Dv=64, T=64, k_bits=4, v_bits=2, dtype="f32", seed=41)
    rng = np.random.default_rng(0)
    K = rng.standard_normal((1, 1, 64, 64)).astype(np.float32)
    V = rng.standard_normal((1, 1, 64, 64)).astype(np.float32)
    K[:, :, :32, 5] = 1.25
    K[:, :, :32, 6] = -0.0
    K[:, :, 32:, 7] = 0.0
    K[:, :, 32:, 7][:, :, ::2] = -0.0
    V[:, :, 3, :32] = -3.5
    V[:, :, 4, 32:] = -0.0
    lay = api.Layout.from_workload(w)
    cache = api.kv_quant_pack(lay, to_device(K, "f32"), to_device(V, "f32"))
    torch.cuda.synchronize()
    _compare_pack(cache_to_numpy(cache), O.pack_all(K, V, w))


@pytest.mark.parametrize("D", [64, 128])
def test_pack_rounding_ties_and_near_ties(D):
    """Quotients (x - z) / s exactly on a half-integer (round half to even) and one
    float32 step either side of it, for every bit width and dtype (head width 128 is
    the 16-bit inputs' dedicated pack kernel): the codes must be the contract's,
    which the kernels get by multiplying with 1/s and falling back to the exact
    division near a rounding boundary."""
    for bits in (2, 4, 8):
        for dtype in ("f32", "bf16", "f16"):
            w = Workload("ties%d_%s_d%d" % (bits, dtype, D), B=1, Hq=4, Hkv=1, Dk=D, Dv=D, T=64, k_bits=bits,
                         v_bits=bits, dtype=dtype, seed=42)
            levels = 2 ** bits - 1
            # s = 1, z = 0 for every group: min 0 and max = levels in each column / row
            grid = np.arange(D, dtype=np.float32) % (levels + 1)
            K = np.zeros((1, 1, 64, D), dtype=np.float32)
            V = np.zeros((1, 1, 64, D), dtype=np.float32)
            for t in range(64):
                K[0, 0, t, :] = (grid + 0.5 * (t % 3 == 1)) % (levels + 0.5)
                V[0, 0, t, :] = (grid + 0.5 * (t % 2)) % (levels + 0.5)
            K[0, 0, 0, :], K[0, 0, 31, :], K[0, 0, 32, :], K[0, 0, 63, :] = 0.0, levels, 0.0, levels
            V[0, 0, :, 0::32], V[0, 0, :, 31::32] = 0.0, levels
            if dtype == "f32":
                # one float32 step below / above a tie on a few elements
                K[0, 0, 4, 1::4] = np.nextafter(K[0, 0, 4, 1::4], np.float32(-1))
                V[0, 0, 5, 2::5] = np.nextafter(V[0, 0, 5, 2::5], np.float32(levels + 1))
                Kin, Vin = K, V
            elif dtype == "bf16":
                Kin = (K.view(np.uint32) >> 16).astype(np.uint16)
                Vin = (V.view(np.uint32) >> 16).astype(np.uint16)
            else:
                Kin = K.astype(np.float16).view(np.uint16)   # every value here is exact in fp16
                Vin = V.astype(np.float16).view(np.uint16)
            lay = api.Layout.from_workload(w)
            cache = api.kv_quant_pack(lay, to_device(Kin, dtype), to_device(Vin, dtype))
            torch.cuda.synchronize()
            _compare_pack(cache_to_numpy(cache), O.pack_all(Kin, Vin, w), w.name + " ")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_pack_ties_with_offset_groups(dtype):
    """Exact half-integer quotients in groups whose minimum is far from zero (z = +-32
    .. +-47), on the 16-bit inputs' 128-wide pack kernel: that kernel forms the fast
    quotient as one fma, x r - z r, whose error grows with |z r|, and widens its
    window of elements that take the exact division to match; the codes must still
    be the contract's (round half to even of fl(fl(x - z) / s)).  Values x = z + k s/2
    with s a power of two, every k from 0 to 2 levels in each group, so that every
    group's range is exactly levels * s and every odd k is a tie."""
    D = 128
    for bits in ((2, 4, 8) if dtype == "f16" else (2, 4)):
        levels = 2 ** bits - 1
        # half-steps s / 2 must be exact in the input format at |x| < 64
        s = 1.0 / 16 if dtype == "f16" else 0.5
        w = Workload("ties_off%d_%s" % (bits, dtype), B=1, Hq=4, Hkv=1, Dk=D, Dv=D, T=64, k_bits=bits, v_bits=bits,
                     dtype=dtype, seed=43)
        K = np.zeros((1, 1, 64, D), dtype=np.float32)
        V = np.zeros((1, 1, 64, D), dtype=np.float32)
        nk = 2 * levels + 1
        for t in range(64):
            for c in range(D):
                zk = (32.0 + (c % 8)) * (1 if c % 3 else -1)
                kk = 0 if t % 32 == 0 else (nk - 1 if t % 32 == 31 else (7 * t + 3 * c) % nk)
                K[0, 0, t, c] = zk + kk * s / 2
                zv = (40.0 + (t % 8)) * (1 if (t + c // 32) % 2 else -1)
                kv = 0 if c % 32 == 0 else (nk - 1 if c % 32 == 31 else (5 * c + 11 * t) % nk)
                V[0, 0, t, c] = zv + kv * s / 2
        if dtype == "f16":
            for x in (K, V):
                assert np.array_equal(x.astype(np.float16).astype(np.float32), x)
            Kin, Vin = K.astype(np.float16).view(np.uint16), V.astype(np.float16).view(np.uint16)
        else:
            assert not (K.view(np.uint32) & 0xFFFF).any() and not (V.view(np.uint32) & 0xFFFF).any()
            Kin = (K.view(np.uint32) >> 16).astype(np.uint16)
            Vin = (V.view(np.uint32) >> 16).astype(np.uint16)
        lay = api.Layout.from_workload(w)
        cache = api.kv_quant_pack(lay, to_device(Kin, dtype), to_device(Vin, dtype))
        torch.cuda.synchronize()
        ref = O.pack_all(Kin, Vin, w)
        # the construction gives s exactly and z exactly (so the ties are real ties)
        for key in ("k_scale", "v_scale"):
            assert np.all(ref[key].view(np.float16).astype(np.float32) == np.float32(s))
        _compare_pack(cache_to_numpy(cache), ref, w.name + " ")


# ------------------------------------------------------------------ full-size runs

def _sample_slabs(w, n):
    rng = np.random.default_rng(1234)
    picks = {(0, 0), (w.B - 1, w.Hkv - 1)}
    while len(picks) < min(n, w.B * w.Hkv):
        picks.add((int(rng.integers(w.B)), int(rng.integers(w.Hkv))))
    return sorted(picks)


def _full_size(w: Workload, n_slabs: int):
    _log("full-size %s: generating and uploading" % w.name)
    Kd, Vd, qd = upload_workload(w)
    lay = api.Layout.from_workload(w)
    _log("full-size %s: pack" % w.name)
    cache = api.kv_quant_pack(lay, Kd, Vd)
    scale = float(O.default_scale(w.Dk))
    plan = api.decode_plan(lay, w.partitions)
    _log("full-size %s: decode P=%d (%s)" % (w.name, w.partitions, plan))
    assert plan["kernel"] == _expected_kernel(w)
    out = api.kv_decode_attn(lay, qd, cache, num_partitions=w.partitions, softmax_scale=scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    G = w.G
    slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)] if n_slabs is None else _sample_slabs(w, n_slabs)
    _log("full-size %s: oracle on %d slabs in worker processes" % (w.name, len(slabs)))
    worst = 0.0
    for b, h, ref, want in slab_references(w.name, slabs, scale):
        gpu = cache_to_numpy({k: t[b, h] for k, t in cache.items()})
        _compare_pack(gpu, ref, "%s slab (%d,%d) " % (w.name, b, h))
        err = np.abs(out[b, h * G:(h + 1) * G] - want).max()
        assert err <= MAX_ABS_ERR, (w.name, b, h, err)
        worst = max(worst, err)
    _log("  %d slabs: packed bytes equal, decode max|err| %.2e" % (len(slabs), worst))
    return Kd, Vd, qd, lay, cache


@pytest.mark.slow
def test_logquant_32k_full_size():
    """Every one of the 256 slabs: packed bytes equal and decode within the bound."""
    _full_size(workload("logquant_32k"), None)


@pytest.mark.slow
def test_thin_keys_16k_full_size():
    """Every one of the 128 slabs."""
    _full_size(workload("thin_keys_16k"), None)


@pytest.mark.slow
def test_long_128k_full_size_and_prefill_chunk():
    """128K-token cache at 64 partitions, then the 8192-token prefill chunk re-packed
    on its own into the same cache must leave every byte unchanged, and that chunk's
    part of the cache equals the oracle's on every slab."""
    w = workload("long_128k")
    Kd, Vd, qd, lay, cache = _full_size(w, None)
    before = {k: v.clone() for k, v in cache.items()}
    t0 = w.T - w.prefill_chunk
    api.kv_quant_pack(lay, Kd[:, :, t0:].contiguous(), Vd[:, :, t0:].contiguous(), cache=cache, t_begin=t0)
    torch.cuda.synchronize()
    for k in cache:
        assert torch.equal(before[k], cache[k]), k
    # The chunk's part of the cache on every slab against the oracle: with a
    # window-only retention the chunk packs like a cache of its own length (its
    # 8064 oldest tokens are the cache's last 252 key groups, its newest 128 the
    # fp16 rows).
    Kc = Kd[:, :, t0:].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    Vc = Vd[:, :, t0:].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    gpu_all = cache_to_numpy(cache)
    nq = w.prefill_chunk - w.n_recent
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = O.pack_slab(Kc[b, h], Vc[b, h], w.dtype, w.k_bits, w.v_bits, w.n_recent, w.log_window)
            gpu = {"k_codes": gpu_all["k_codes"][b, h, -nq:], "k_scale": gpu_all["k_scale"][b, h, -nq // 32:],
                   "k_zero": gpu_all["k_zero"][b, h, -nq // 32:], "v_codes": gpu_all["v_codes"][b, h, -nq // 32:],
                   "v_scale": gpu_all["v_scale"][b, h, -nq // 32:], "v_zero": gpu_all["v_zero"][b, h, -nq // 32:],
                   "k_fp16": gpu_all["k_fp16"][b, h], "v_fp16": gpu_all["v_fp16"][b, h]}
            _compare_pack(gpu, ref, "%s chunk slab (%d,%d) " % (w.name, b, h))
    _log("  prefill chunk: every slab's packed bytes equal the oracle's")


def test_workspace_reuse_needs_no_initialisation():
    """One workspace serves consecutive calls whatever it holds on entry (it is
    filled with garbage first): repeated calls give bit-identical output (the merge
    combines partitions in a fixed order), and a smaller partition count reuses it."""
    w = small_cases()[0]
    K, V = make_all(w, workers=4)
    q = make_queries(w)
    lay = api.Layout.from_workload(w)
    cache = api.kv_quant_pack(lay, to_device(K, w.dtype), to_device(V, w.dtype))
    qd = to_device(q, w.dtype)
    ws = api.alloc_workspace(lay, 7)
    ws.fill_(0xA5)
    scale = float(O.default_scale(w.Dk))
    want = O.decode_all(q, O.pack_all(K, V, w), w, scale)
    outs = []
    for P in (7, 7, 3, 7):
        out = api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale, workspace=ws)
        torch.cuda.synchronize()
        err = np.abs(out.cpu().numpy().astype(np.float64) - want).max()
        assert err <= MAX_ABS_ERR, (P, err)
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[3])


@pytest.mark.parametrize("name,kernel", [("small_k4v2_win", "mfma"), ("small_k4v8_f32", "valu")])
def test_timed_decode_events(name, kernel):
    """kv_decode_attn_timed: the same output bits as kv_decode_attn, with its two
    events as the start and stop events of the decode kernel: a positive interval that
    lies inside events recorded around the whole call, for both decode kernels, at
    P = 1 (no merge) and at the configured P."""
    w = {c.name: c for c in small_cases()}[name]
    K, V = make_all(w, workers=4)
    q = make_queries(w)
    lay = api.Layout.from_workload(w)
    cache = api.kv_quant_pack(lay, to_device(K, w.dtype), to_device(V, w.dtype))
    qd = to_device(q, w.dtype)
    scale = float(O.default_scale(w.Dk))
    want = O.decode_all(q, O.pack_all(K, V, w), w, scale)
    for P in (1, w.partitions):
        plan = api.decode_plan(lay, P)
        assert plan["kernel"] == kernel, (name, P, plan)
        plain = api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in ev:
            e.record()
        torch.cuda.synchronize()
        ev[0].record()
        timed = api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale,
                                   kernel_events=(ev[1], ev[2]))
        ev[3].record()
        torch.cuda.synchronize()
        assert torch.equal(plain.cpu(), timed.cpu()), (name, P)
        err = np.abs(timed.cpu().numpy().astype(np.float64) - want).max()
        assert err <= MAX_ABS_ERR, (name, P, err)
        kern, call = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
        before, after = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
        _log("%s P=%d kernel %.1f us, call %.1f us" % (name, P, kern * 1e3, call * 1e3))
        assert 0 < kern <= call and before >= 0 and after >= 0, (name, P, kern, call, before, after)


@pytest.mark.gpu
def test_read_probe_runs():
    """The measurement probe reads a buffer (with a tail that is not a whole
    workgroup block) and leaves it untouched."""
    dev = torch.device("cuda:0")
    buf = torch.arange((1 << 20) + 12, dtype=torch.int32, device=dev)
    ref = buf.clone()
    api.kvq_read_probe(buf)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
