"""Oracle pack and decode of whole (batch, KV head) slabs of a named workload, one
slab per task, for the full-size GPU tests, which spread them over worker processes
so that every slab can be compared.  Test infrastructure: numpy and the oracle only
(no torch, no GPU)."""

import os


def slab_reference(args):
    """(workload name, b, h, softmax scale) -> (b, h, packed slab, decode output of
    the slab's query heads) from the oracle, on the workload's seeded inputs."""
    name, b, h, scale = args
    import oracle as O
    from workloads import make_queries, make_slab, workload
    w = workload(name)
    s = make_slab(w, b, h)
    ref = O.pack_slab(s.K, s.V, w.dtype, w.k_bits, w.v_bits, w.n_recent, w.log_window)
    q = make_queries(w)
    want = O.decode_slab(q[b, h * w.G:(h + 1) * w.G], ref, w.dtype, w.k_bits, w.v_bits, scale)
    return b, h, ref, want


def _one_blas_thread():
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"


def slab_references(name, slabs, scale, max_workers=16):
    """Yields slab_reference results for every (b, h) of `slabs`, computed in spawned
    worker processes (the calling process may hold the GPU; the workers do not touch it)."""
    import multiprocessing as mp
    workers = max(1, min(max_workers, len(os.sched_getaffinity(0)), len(slabs)))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_one_blas_thread) as pool:
        yield from pool.imap_unordered(slab_reference, [(name, b, h, scale) for b, h in slabs])
