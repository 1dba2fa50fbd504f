"""Benchmark of the packed-KV decode hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input on the
128K-token workload (B=4, 32 query / 8 KV heads, head dim 128, K4V2, 128-token fp16
window):  kv_quant_pack of the newest 8192-token prefill chunk into its place in
the packed cache, then kv_decode_attn of one new token per sequence over all
131072 cached tokens with 64 split-K partitions.  Inputs are resident in HBM
before timing starts.

Prints one JSON line.  ``value`` is the effective HBM throughput of a whole step:
the algorithmic bytes of the step (each packed byte, scale, zero, fp16 row, query
and output moved once; the prefill chunk read once and its packed form written
once) divided by the measured step time.

Beside the step (not part of ``value``), the ``configs`` object times decode alone on
the other workloads of the list (the Llama-8B-shaped 4096-token cache, the 32K-token
cache with log-spaced fp16 tokens and the thin-key 16K-token cache), each call after
an untimed cache-evicting read, with its own roofline and CPU baseline; the
``valu_variants`` object times the formats that decode on the vector-ALU kernel
(1- and 3-bit codes, the HeadQ side code) at the 128K shape; the ``stream`` object times the streaming
cache at the same shape: after a prefill to just under the full length, decode
steps that append one token per sequence (kv_stream_append) and then attend over
the stream (kv_stream_decode), each call bracketed by events; the
``format_variants`` object times decode at the same shape with keys in groups of
32 or 128 tokens and values in groups of 32, 64 or 128 channels (fewer scale and
zero bytes), the caches' calls interleaved one by one.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak, 8 TB/s
METRIC = "quantized-KV decode attn: effective HBM GB/s (% of peak) + decode steps/sec"
CSRC = os.path.join(ROOT, "quantized_decode_attention_kv_amd", "csrc")
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("kvq_decode_mfma.hip", "kvq_decode_common.hpp", "kvq_decode_generic.hip",
                                                "kvq_decode_merge.hip", "kvq_internal.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_long_128k_hbm_traffic.txt")


# ----------------------------------------------------------------- byte accounting

def decode_bytes(w, R, Tq):
    """Algorithmic bytes of one decode call: packed codes, scales and zeros, fp16
    retained rows, the queries (storage dtype) and the float32 output, each once."""
    slabs = w.B * w.Hkv
    qb = 4 if w.dtype == "f32" else 2
    k_codes = slabs * Tq * w.Dk * w.k_bits // 8
    k_sz = slabs * (Tq // w.k_group) * w.Dk * 2 * 2
    v_codes = slabs * Tq * w.Dv * w.v_bits // 8
    v_sz = slabs * Tq * (w.Dv // w.v_group) * 2 * 2
    fp16 = slabs * R * (w.Dk + w.Dv) * 2
    return k_codes + k_sz + v_codes + v_sz + fp16 + w.B * w.Hq * w.Dk * qb + w.B * w.Hq * w.Dv * 4


def pack_bytes(w, n_tokens, n_quant):
    """Algorithmic bytes of packing n_tokens positions of which n_quant are quantized:
    K and V read once, codes / scales / zeros / fp16 rows written once."""
    slabs = w.B * w.Hkv
    eb = 4 if w.dtype == "f32" else 2
    read = slabs * n_tokens * (w.Dk + w.Dv) * eb
    n_ret = n_tokens - n_quant
    write = (slabs * n_quant * (w.Dk * w.k_bits + w.Dv * w.v_bits) // 8
             + slabs * (n_quant // w.k_group) * w.Dk * 4 + slabs * n_quant * (w.Dv // w.v_group) * 4
             + slabs * n_ret * (w.Dk + w.Dv) * 2)
    return read + write


def kernel_source_hash():
    """Hash of the decode kernel sources without their comments and blank lines, to
    tell whether stored counter data is current (a comment edit changes no kernel)."""
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for line in text.splitlines():
            code = re.sub(r"//.*", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def _profile_value(path, key):
    """A figure ``key: value`` of a committed profile summary, if the summary was taken
    on the current decode kernel source (else None)."""
    try:
        text = open(path).read()
    except OSError:
        return None
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"%s:\s*([0-9.eE+]+)" % re.escape(key), text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def read_traffic(name="long_128k"):
    """HBM bytes per decode launch on a workload from the committed counter summary,
    if it was taken on the current decode kernel source (else None)."""
    path = TRAFFIC_FILE if name == "long_128k" else os.path.join(ROOT, "profiles", "decode_%s_hbm_traffic.txt" % name)
    return _profile_value(path, "hbm_bytes_per_launch")


def read_rocprof_us(name):
    """Mean decode-kernel duration (us) that rocprofv3 measured on a workload, from the
    committed kernel-trace summary, if taken on the current decode source (else None)."""
    return _profile_value(os.path.join(ROOT, "profiles", "decode_%s_kernel_trace.txt" % name), "decode_kernel_avg_us")


# ------------------------------------------------------------------ CPU baseline

def _cpu_worker(args):
    """Runs in a spawned process: oracle on a list of (b, h) slabs of the workload.
    Returns (seconds spent in the oracle, bytes covered)."""
    wname, v_group, k_group, slabs = args
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    import numpy as np
    import oracle as O
    from workloads import make_queries, make_slab, workload
    w = workload(wname).with_(v_group=v_group, k_group=k_group)
    q = make_queries(w)
    t_chunk = w.T - w.prefill_chunk
    spent = 0.0
    for b, h in slabs:
        s = make_slab(w, b, h)
        # the packed cache before the step (setup, not timed)
        full = O.pack_slab(s.K, s.V, w.dtype, w.k_bits, w.v_bits, w.n_recent, w.log_window, v_group=w.v_group,
                           k_group=w.k_group)
        t0 = time.perf_counter()
        # the step: pack the prefill chunk ...
        if w.prefill_chunk:
            _oracle_pack_chunk(O, s, w, t_chunk)
        # ... and decode the G query heads of this kv head over the whole slab
        G = w.Hq // w.Hkv
        O.decode_slab(q[b, h * G:(h + 1) * G], full, w.dtype, w.k_bits, w.v_bits, O.default_scale(w.Dk))
        spent += time.perf_counter() - t0
    return spent, len(slabs)


def _oracle_pack_chunk(O, s, w, t0):
    """Oracle pack of positions [t0, T) of a slab.  With a recent window only (no
    log-spaced positions) the chunk's retained tokens are its newest ones and the
    rest are whole key groups, so the chunk packs like a cache of its own length."""
    assert w.log_window == 0
    n = w.T - t0
    return O.pack_slab(s.K[t0:], s.V[t0:], w.dtype, w.k_bits, w.v_bits, min(w.n_recent, n), 0, v_group=w.v_group,
                       k_group=w.k_group)


def cpu_baseline(w, step_bytes, budget_workers=None, max_workers=16):
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    cores = budget_workers or max(1, min(max_workers, affinity))
    slabs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    per = [slabs[i::cores] for i in range(cores)]
    per = [p[:1] for p in per if p]          # one slab per worker: about 1-2 s of oracle work each
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(len(per)) as pool:
        res = pool.map(_cpu_worker, [(w.name, w.v_group, w.k_group, p) for p in per])
    wall = time.perf_counter() - t0
    busiest = max(r[0] for r in res)
    n_slabs = sum(r[1] for r in res)
    covered = step_bytes * n_slabs / (w.B * w.Hkv)
    return {
        "value": covered / busiest / 1e9,
        "unit": "GB/s",
        "cores": len(per),
        "host_cpus": affinity,
        "kind": "oracle",
        "sample": ("%d of %d (batch, kv-head) slabs of the step, one per worker process (1 BLAS thread each): "
                   "%sfloat64 decode over the whole %d-token slab; throughput = the slabs' share of the step's "
                   "algorithmic bytes / the busiest worker's oracle time (%.2f s; %.1f s wall incl. input "
                   "generation and the untimed full-slab pack; workers capped at %d of the host's %d CPUs)"
                   % (n_slabs, w.B * w.Hkv,
                      ("oracle pack of the %d-token prefill chunk + " % w.prefill_chunk) if w.prefill_chunk else "",
                      w.T, busiest, wall, max_workers, affinity)),
    }


# ------------------------------------------------------------------------- main

def read_ceiling(torch, api, nbytes, dev, reps=20):
    """HBM read rate of a plain grid-wide streaming read (kvq_read_probe) over
    nbytes, median of reps calls (after the timed steps; not part of them)."""
    buf = torch.zeros((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=dev)
    sink = torch.empty(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        api.kvq_read_probe(buf, sink)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        api.kvq_read_probe(buf, sink)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    med = ts[len(ts) // 2]
    del buf
    return {"read_GBps": round(nbytes / (med * 1e-3) / 1e9, 1), "us": round(med * 1e3, 2), "bytes": nbytes,
            "how": "kvq_read_probe: grid-wide streaming read of the decode's byte count, median of %d calls" % reps}


def stream_setup(torch, api, w, Kd, Vd, n_steps):
    """A streaming cache at the workload's shape, prefilled to the longest length
    (<= T - n_steps) whose quantized count is a multiple of 32, and the K/V rows of
    the n_steps tokens that follow (one contiguous [B, Hkv, D] tensor each)."""
    T0 = w.T - n_steps
    while T0 > 0:
        try:
            api.Layout(w.B, w.Hq, w.Hkv, w.Dk, w.Dv, T0, w.k_bits, w.v_bits, min(w.n_recent, T0), w.log_window)
            break
        except api.L_.KvqError:
            T0 -= 1
    s = api.Stream(w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T, w.k_bits, w.v_bits, w.n_recent, w.log_window)
    s.prefill(Kd[:, :, :T0].contiguous(), Vd[:, :, :T0].contiguous())
    toks = [(Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous()) for t in range(T0, T0 + n_steps)]
    torch.cuda.synchronize()
    return {"s": s, "T0": T0, "toks": toks}


def stream_run(torch, st, qd, P, scale):
    """Decode steps on the streaming cache: append one token per sequence, then
    attend over the stream.  Events bracket each call on the current stream, so an
    append's time includes the host-side planning and launch of that call (the GPU
    waits for it)."""
    s, toks = st["s"], st["toks"]
    n = len(toks)
    ws = torch.empty(max(16, s.workspace_bytes(P)), dtype=torch.uint8, device=qd.device)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.float32, device=qd.device)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    formed = []
    torch.cuda.synchronize()
    host = 0.0
    for i, (k, v) in enumerate(toks):
        g0 = s.n_groups
        ev[i][0].record()
        h0 = time.perf_counter()
        s.append(k, v)
        host += time.perf_counter() - h0
        ev[i][1].record()
        s.decode(qd, num_partitions=P, softmax_scale=scale, out=out, workspace=ws)
        ev[i][2].record()
        formed.append(s.n_groups > g0)
    torch.cuda.synchronize()
    app = [e[0].elapsed_time(e[1]) for e in ev]
    dec = [e[1].elapsed_time(e[2]) for e in ev]
    with_group = [a for a, f in zip(app, formed) if f]
    plain = [a for a, f in zip(app, formed) if not f]
    return {
        "prefill_tokens": st["T0"], "decode_steps": n, "groups_formed": len(with_group),
        "tokens_after": s.t, "fp16_rows": s.n_rows,
        "append_us_p10_p50_p90": percentiles(plain),
        "append_with_group_us_p10_p50_p90": percentiles(with_group) if with_group else None,
        "append_host_us_per_call": round(host * 1e6 / n, 2),
        "decode_us_p10_p50_p90": percentiles(dec),
        "step_us_mean": round(sum(a + d for a, d in zip(app, dec)) * 1e3 / n, 2),
    }


FORMAT_VARIANTS = [(32, 32), (32, 64), (32, 128), (128, 32), (128, 128)]   # (k_group, v_group)


def variants_setup(api, w, Kd, Vd, lay, cache):
    """Caches of the full workload with keys in groups of 32 or 128 tokens and values
    in groups of 32, 64 or 128 channels (where the shape allows); the step's own cache
    serves its own format."""
    out = {}
    for kg, vg in FORMAT_VARIANTS:
        wv = w.with_(k_group=kg, v_group=vg)
        if (kg, vg) == (w.k_group, w.v_group):
            out[(kg, vg)] = (lay, cache)
            continue
        try:
            lv = api.Layout.from_workload(wv)
        except api.L_.KvqError:
            continue   # this shape's quantized count is not a multiple of the key group
        out[(kg, vg)] = (lv, api.kv_quant_pack(lv, Kd, Vd))
    return out


def variants_run(torch, api, w, variants, qd, P, scale, reps=30):
    """Decode over each format variant, calls interleaved one by one so that all see
    the same clock and thermal state; the start and stop events of each decode
    kernel's launch."""
    ws = {key: api.alloc_workspace(lv, P, qd.device) for key, (lv, _) in variants.items()}
    out = torch.empty((w.B, w.Hq, w.Dv), dtype=torch.float32, device=qd.device)
    ev = {key: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)] for key in variants}
    for key in variants:
        for e in ev[key]:
            for x in e:
                x.record()
    torch.cuda.synchronize()
    for i in range(reps):
        for key, (lv, c) in variants.items():
            api.kv_decode_attn(lv, qd, c, num_partitions=P, softmax_scale=scale, out=out, workspace=ws[key],
                               kernel_events=(ev[key][i][0], ev[key][i][1]))
    torch.cuda.synchronize()
    res = {}
    for (kg, vg), (lv, _) in variants.items():
        ts = [e[0].elapsed_time(e[1]) for e in ev[(kg, vg)]]
        p = percentiles(ts)
        db = decode_bytes(w.with_(k_group=kg, v_group=vg), lv.R, lv.Tq)
        res["k%d_v%d" % (kg, vg)] = {"decode_kernel_us_p10_p50_p90": p, "algorithmic_bytes": db,
                                     "GBps_at_p50": round(db / (p[1] * 1e-6) / 1e9, 1)}
    return res


def decode_cold(torch, api, lay, cache, qd, P, scale, dev, reps=20):
    """Decode kernel time with nothing of the cache left in the caches: before each
    call an untimed plain read of 1 GiB (four times the 256 MB memory-side cache)
    evicts it.  A read, not a write: freshly written lines would be written back
    inside the decode.  The read is a torch reduction (plain loads that allocate in
    the caches), not kvq_read_probe, whose loads carry the non-temporal hint.
    Events bracket the decode kernel and the whole call."""
    flush = torch.zeros(1 << 27, dtype=torch.int64, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)
    ws = api.alloc_workspace(lay, P, dev)
    out = torch.empty((lay.B, lay.Hq, lay.Dv), dtype=torch.float32, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(2 * reps)]
    for e in ev:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    # alternate calls: the kernel's own events on one, events around a plain call
    # on the next (a timed launch costs the call a few microseconds)
    for i in range(2 * reps):
        torch.sum(flush, dim=0, out=sink)
        if i % 2 == 0:
            api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale, out=out, workspace=ws,
                               kernel_events=(ev[i][0], ev[i][1]))
        else:
            ev[i][0].record()
            api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale, out=out, workspace=ws)
            ev[i][1].record()
    torch.cuda.synchronize()
    del flush
    kern = [e[0].elapsed_time(e[1]) for e in ev[0::2]]
    call = [e[0].elapsed_time(e[1]) for e in ev[1::2]]
    return {"kernel_us_p10_p50_p90": percentiles(kern), "kernel_us_mean": round(sum(kern) * 1e3 / reps, 2),
            "call_us_p10_p50_p90": percentiles(call), "call_us_mean": round(sum(call) * 1e3 / reps, 2),
            "how": "1 GiB untimed read before each of 2 x %d calls; kernel: the decode kernel's start and stop "
                   "events (hipExtLaunchKernel) on every other call, call: events around the other, plain calls"
                   % reps}


def decode_back_to_back(torch, api, lay, cache, qd, P, scale, dev, reps=20):
    """Decode kernel time with the calls back to back (no read in between; the
    previous call's lines are all that the caches can hold).  Sustained back-to-back
    load can lower the clocks, which the spread of these times shows."""
    ws = api.alloc_workspace(lay, P, dev)
    out = torch.empty((lay.B, lay.Hq, lay.Dv), dtype=torch.float32, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for i in range(reps):
        api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale, out=out, workspace=ws,
                           kernel_events=(ev[i][0], ev[i][1]))
    torch.cuda.synchronize()
    kern = [e[0].elapsed_time(e[1]) for e in ev]
    return {"kernel_us_p10_p50_p90": percentiles(kern), "kernel_us_mean": round(sum(kern) * 1e3 / reps, 2),
            "how": "%d calls back to back, the start and stop events of each decode kernel's launch" % reps}


# Decode alone on the other workloads of the list (each its own cache).
DECODE_CONFIGS = ["llama8b_gqa_4k", "logquant_32k", "thin_keys_16k"]


def describe(w, P):
    return ("%s: B%d Hq%d Hkv%d Dk%d Dv%d T%d K%dV%d fp16-window %d log-window %d, %d partitions"
            % (w.name, w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T, w.k_bits, w.v_bits, w.n_recent, w.log_window, P))


def decode_config(torch, api, name, dev, reps, with_cpu):
    """Decode on one workload: cache packed once (untimed), then calls timed after a
    cache-evicting read (decode_cold); roofline of the decode kernel from the mean
    event time, beside rocprofv3's mean from the committed summary when current."""
    from workloads import workload
    from workloads.device import upload_workload
    w = workload(name)
    P = w.partitions
    print("# %s: generating inputs" % name, file=sys.stderr, flush=True)
    Kd, Vd, qd = upload_workload(w)
    lay = api.Layout.from_workload(w)
    cache = api.kv_quant_pack(lay, Kd, Vd)
    del Kd, Vd
    plan = api.decode_plan(lay, P)
    scale = 1.0 / (w.Dk ** 0.5)
    for _ in range(3):
        api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale)
    torch.cuda.synchronize()
    print("# %s: decode, %d cold calls" % (name, reps), file=sys.stderr, flush=True)
    cold = decode_cold(torch, api, lay, cache, qd, P, scale, dev, reps)
    print("# %s: decode, %d calls back to back" % (name, reps), file=sys.stderr, flush=True)
    b2b = decode_back_to_back(torch, api, lay, cache, qd, P, scale, dev, reps)
    db = decode_bytes(w, lay.R, lay.Tq)
    kern_us = cold["kernel_us_mean"]
    call_us = cold["call_us_mean"]
    achieved = db / (kern_us * 1e-6) / 1e9
    rp_us = read_rocprof_us(name)
    res = {
        "workload": describe(w, P),
        "plan": plan,
        "algorithmic_bytes": db,
        "decode": {"kernel": cold, "back_to_back": b2b, "GBps_call": round(db / (call_us * 1e-6) / 1e9, 1),
                   "steps_per_s": round(1e6 / call_us, 1), "tokens_per_s": round(w.B * 1e6 / call_us, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": read_traffic(name),
                     "kernel": "decode_%s_kernel (first kernel of kv_decode_attn)" % plan["kernel"],
                     "kernel_us": kern_us,
                     "timing": "HIP start and stop events of the decode kernel's launch (hipExtLaunchKernel), "
                               "mean over the cold calls",
                     "rocprof_kernel_us": rp_us,
                     "frac_rocprof": None if rp_us is None else round(db / (rp_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)},
    }
    del cache
    torch.cuda.empty_cache()
    if with_cpu:
        print("# %s: cpu baseline (oracle)" % name, file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, db)
    return res


def valu_setup(torch, api, w, Kd, Vd, dev):
    """Caches of the formats that decode on the vector-ALU kernel, at the workload's
    shape: 1- and 3-bit codes and the HeadQ side code (rank 8, 8-bit side codes, a
    random orthonormal basis per KV head), next to K4V4 on the matrix-core kernel.
    Each is packed once (untimed set-up)."""
    import numpy as np
    caches = {}
    for name, kb, vb in (("k1v1", 1, 1), ("k3v3", 3, 3), ("k4v4", 4, 4)):
        wv = w.with_(k_bits=kb, v_bits=vb)
        lv = api.Layout.from_workload(wv)
        caches[name] = (wv, lv, api.kv_quant_pack(lv, Kd, Vd), None)
    rank = 8
    rng = np.random.default_rng(7)
    U = np.stack([np.linalg.qr(rng.standard_normal((w.Dk, rank)))[0] for _ in range(w.Hkv)]).astype(np.float32)
    Ud = torch.from_numpy(U).to(dev)
    ls = api.Layout.from_workload(w)
    cs = api.kv_quant_pack(ls, Kd, Vd)
    side = api.side_pack(ls, Kd, cs, Ud, side_bits=8)
    caches["k%dv%d_side_r%d" % (w.k_bits, w.v_bits, rank)] = (w, ls, cs, (Ud, side))
    return caches


def valu_run(torch, api, w, caches, qd, P, scale, dev, reps=10):
    """Decode over each cache of valu_setup, calls interleaved one by one; events
    around each call (decode kernel and merge)."""
    rank = 8
    out = torch.empty((w.B, w.Hq, w.Dv), dtype=torch.float32, device=dev)
    ev = {k: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)] for k in caches}
    for k in caches:
        for e in ev[k]:
            e[0].record()
            e[1].record()
    torch.cuda.synchronize()
    for i in range(reps):
        for k, (wv, lv, c, sd) in caches.items():
            ev[k][i][0].record()
            if sd is None:
                api.kv_decode_attn(lv, qd, c, num_partitions=P, softmax_scale=scale, out=out)
            else:
                api.kv_decode_attn_side(lv, qd, c, sd[0], sd[1], num_partitions=P, softmax_scale=scale)
            ev[k][i][1].record()
    torch.cuda.synchronize()
    res = {}
    for k, (wv, lv, c, sd) in caches.items():
        ts = [e[0].elapsed_time(e[1]) for e in ev[k]]
        p = percentiles(ts)
        db = decode_bytes(wv, lv.R, lv.Tq)
        if sd is not None:   # side codes (one byte each), their fp16 scale and zero, and the basis
            db += w.B * w.Hkv * lv.Tq * (rank + 4) + w.Hkv * w.Dk * rank * 4
        res[k] = {"kernel": api.decode_plan(lv, P, side_code=sd is not None)["kernel"],
                  "decode_call_us_p10_p50_p90": p, "algorithmic_bytes": db,
                  "GBps_at_p50": round(db / (p[1] * 1e-6) / 1e9, 1)}
    return res


def percentiles(xs):
    xs = sorted(xs)
    pick = lambda f: xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]
    return [round(pick(0.1) * 1e3, 2), round(pick(0.5) * 1e3, 2), round(pick(0.9) * 1e3, 2)]


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_128k",
                    help="workload name (the headline step is long_128k; others are for exploration)")
    ap.add_argument("--partitions", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming-cache leg")
    ap.add_argument("--stream-steps", type=int, default=256)
    ap.add_argument("--event-every", type=int, default=4,
                    help="record the decode-timing events on every n-th timed step only (each event delays the "
                         "next kernel by a few microseconds)")
    ap.add_argument("--no-variants", action="store_true", help="skip the format-variants leg")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-cold decode leg")
    ap.add_argument("--no-valu", action="store_true", help="skip the vector-ALU formats leg")
    ap.add_argument("--no-configs", action="store_true", help="skip the decode legs of the other workloads")
    ap.add_argument("--configs", default=",".join(DECODE_CONFIGS),
                    help="comma-separated workloads of the decode-only legs")
    ap.add_argument("--config-reps", type=int, default=30, help="timed cold calls per decode-only leg")
    ap.add_argument("--v-group", type=int, default=None, help="channels per value group of the step (default 32)")
    ap.add_argument("--k-group", type=int, default=None, help="tokens per key group of the step (default 32)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU mode (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_decode_attention_kv_amd import api
    from workloads import workload
    from workloads.device import upload_workload

    w = workload(args.workload)
    if args.v_group:
        w = w.with_(v_group=args.v_group)
    if args.k_group:
        w = w.with_(k_group=args.k_group)
    P = args.partitions or w.partitions
    lay = api.Layout.from_workload(w)
    dev = torch.device("cuda:0")
    print("# %s: generating inputs" % w.name, file=sys.stderr, flush=True)
    Kd, Vd, qd = upload_workload(w)
    cache = api.alloc_cache(lay, dev)
    # the cache before the step: everything packed once (untimed setup)
    api.kv_quant_pack(lay, Kd, Vd, cache=cache)
    chunk = w.prefill_chunk
    t0 = w.T - chunk
    if chunk:
        Kc = Kd[:, :, t0:].contiguous()
        Vc = Vd[:, :, t0:].contiguous()
    stream = None if args.no_stream else stream_setup(torch, api, w, Kd, Vd, args.stream_steps)
    variants = None if args.no_variants else variants_setup(api, w, Kd, Vd, lay, cache)
    valu = None if args.no_valu else valu_setup(torch, api, w, Kd, Vd, dev)
    del Kd, Vd
    ws = api.alloc_workspace(lay, P, dev)
    out = torch.empty((w.B, w.Hq, w.Dv), dtype=torch.float32, device=dev)
    scale = 1.0 / (w.Dk ** 0.5)
    torch.cuda.synchronize()

    # Events on the stream the kernels run on.  The timed steps carry only the two
    # the roofline needs, the start and stop events of the decode kernel's launch
    # (hipExtLaunchKernel); the pack and merge are timed in a separate breakdown pass right
    # after, with four events recorded between the kernels (each such record costs
    # the step a few microseconds).
    def step(ev=None, full=False):
        if full:
            ev[0].record()
        if chunk:
            api.kv_quant_pack(lay, Kc, Vc, cache=cache, t_begin=t0)
        if full:
            ev[1].record()
            api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale, out=out, workspace=ws,
                               after_decode_event=ev[2])
            ev[3].record()
        else:
            # ev[1], ev[2]: the start and stop events of the decode kernel's launch
            api.kv_decode_attn(lay, qd, cache, num_partitions=P, softmax_scale=scale, out=out, workspace=ws,
                               kernel_events=None if ev is None else (ev[1], ev[2]))

    def new_events(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for e in evs:
            for x in e:
                x.record()  # torch creates an event at its first record: not inside a timed region
        torch.cuda.synchronize()
        return evs

    print("# %s: warmup %d" % (w.name, args.warmup), file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    # A timed launch may hold the next kernel back a little, so only every
    # event_every-th timed step carries the two decode events; the others run as
    # they would in a decode loop.
    ev_steps = list(range(0, args.steps, max(1, args.event_every)))
    events = new_events(len(ev_steps))
    ev_of = {s: events[k] for k, s in enumerate(ev_steps)}
    start = time.perf_counter()
    for i in range(args.steps):
        step(ev_of.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - start
    kern_ms = sum(e[1].elapsed_time(e[2]) for e in events) / len(events)
    n_bd = min(args.steps, 20)
    bd = new_events(n_bd)
    for i in range(n_bd):
        step(bd[i], full=True)
    torch.cuda.synchronize()
    pack_ms = sum(e[0].elapsed_time(e[1]) for e in bd) / n_bd
    dec_ms = sum(e[1].elapsed_time(e[3]) for e in bd) / n_bd
    gap_kern_ms = sum(e[1].elapsed_time(e[2]) for e in bd) / n_bd
    merge_ms = sum(e[2].elapsed_time(e[3]) for e in bd) / n_bd
    ms_per_step = wall * 1e3 / args.steps

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    n_quant_chunk = lay.quantized_before(w.T) - lay.quantized_before(t0) if chunk else 0
    db = decode_bytes(w, lay.R, lay.Tq)
    pb = pack_bytes(w, chunk, n_quant_chunk) if chunk else 0
    step_bytes = db + pb
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_gbps = db / (dec_ms * 1e-3) / 1e9
    kern_gbps = db / (kern_ms * 1e-3) / 1e9
    traffic = read_traffic()
    rp_us = read_rocprof_us(w.name) if (w.k_group, w.v_group) == (32, 32) and args.partitions is None else None
    ceiling = read_ceiling(torch, api, db, dev)
    cold = None if args.no_cold else decode_cold(torch, api, lay, cache, qd, P, scale, dev)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_detail": "float32 accumulation and softmax; the matrix-core products take fp16 operands, codes exact "
                        "and the folded scales q*s and p*s split into fp16 hi + lo parts (about 22 significant bits)",
        "data": "synthetic: seeded N(0,1) keys with 4 outlier channels x8 and per-channel N(0,2) offsets, "
                "N(0,0.5) values, N(0,1) queries; bf16 in HBM",
        "config": {
            "workload": "%s: B%d Hq%d Hkv%d Dk%d Dv%d T%d K%dV%d fp16-window %d log-window %d, %d partitions%s%s"
                        % (w.name, w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T, w.k_bits, w.v_bits, w.n_recent,
                           w.log_window, P, (", + %d-token prefill pack" % chunk) if chunk else "",
                           (", value groups of %d channels" % w.v_group) if w.v_group != 32 else "")
                        + ((", key groups of %d tokens" % w.k_group) if w.k_group != 32 else ""),
            "batch": w.B, "cached_tokens": w.T, "partitions": P,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "steps_per_s": round(1e3 / ms_per_step, 1),
        "decode": {"us": round(dec_ms * 1e3, 2), "GBps": round(dec_gbps, 1),
                   "pct_of_hbm_peak": round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
                   "steps_per_s": round(1e3 / dec_ms, 1), "tokens_per_s": round(w.B * 1e3 / dec_ms, 1),
                   "kernel_us": round(kern_ms * 1e3, 2), "merge_us": round(merge_ms * 1e3, 2),
                   "kernel_us_with_dispatch_gap": round(gap_kern_ms * 1e3, 2),
                   "kernel_us_p10_p50_p90": percentiles([e[1].elapsed_time(e[2]) for e in events]),
                   "cold": cold, "algorithmic_bytes": db},
        "pack": ({"us": round(pack_ms * 1e3, 2), "GBps": round(pb / (pack_ms * 1e-3) / 1e9, 1),
                  "us_p10_p50_p90": percentiles([e[0].elapsed_time(e[1]) for e in bd]),
                  "algorithmic_bytes": pb} if chunk else None),
        "hbm_read_ceiling": ceiling,
        "roofline": {"bound": "hbm", "achieved": round(kern_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(kern_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": "decode_mfma_kernel (first kernel of kv_decode_attn)",
                     "kernel_us": round(kern_ms * 1e3, 2),
                     "timing": "HIP start and stop events of the decode kernel's launch (hipExtLaunchKernel), "
                               "mean over %d of the %d timed steps (every %d-th); with the dispatch gap "
                               "before it (events around the call, breakdown pass): decode.kernel_us_with_dispatch_gap"
                               % (len(events), args.steps, max(1, args.event_every)),
                     "rocprof_kernel_us": rp_us,
                     "frac_rocprof": None if rp_us is None else round(db / (rp_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "kernel_source_sha256_16": kernel_source_hash()},
    }
    if stream is not None:
        print("# %s: streaming cache, %d decode steps" % (w.name, args.stream_steps), file=sys.stderr, flush=True)
        result["stream"] = stream_run(torch, stream, qd, P, scale)
    if variants is not None:
        print("# %s: format variants" % w.name, file=sys.stderr, flush=True)
        result["format_variants"] = variants_run(torch, api, w, variants, qd, P, scale)
    if valu is not None:
        print("# %s: vector-ALU formats" % w.name, file=sys.stderr, flush=True)
        result["valu_variants"] = valu_run(torch, api, w, valu, qd, P, scale, dev)
    del cache, variants, valu, stream, ws
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = {}
        for name in [c for c in args.configs.split(",") if c and c != w.name]:
            result["configs"][name] = decode_config(torch, api, name, dev, args.config_reps,
                                                    not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        print("# %s: cpu baseline (oracle)" % w.name, file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, step_bytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
