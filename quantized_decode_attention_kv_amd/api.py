"""Python binding of libkvq: argument marshalling only.

PyTorch provides device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  Names follow include/kvq.h.
"""

import ctypes
import math
import types

import torch

from . import _lib as L_

_DTYPE_CODES = {torch.float32: L_.KVQ_F32, torch.float16: L_.KVQ_F16, torch.bfloat16: L_.KVQ_BF16}


class Layout:
    """Shape and fp16-retention policy of one packed cache (kvq_layout)."""

    def __init__(self, B, Hq, Hkv, Dk, Dv, T, k_bits, v_bits, n_recent=0, log_window=0, v_group=32, k_group=32,
                 key_rotation=False):
        lib = L_.load()
        self._c = L_.KvqLayout()
        L_.check(lib.kvq_layout_init_ex(ctypes.byref(self._c), B, Hq, Hkv, Dk, Dv, T, k_bits, v_bits,
                                        n_recent, log_window, k_group, v_group))
        if key_rotation:
            L_.check(lib.kvq_layout_set_flags(ctypes.byref(self._c), L_.KVQ_KEY_ROTATION))
        # the fields never change after this point: plain attributes, so that the
        # per-call wrappers read them without a lookup into the struct
        self.__dict__.update({f: getattr(self._c, f) for f in L_.LAYOUT_FIELDS})
        self.ref = ctypes.byref(self._c)
        self._ws = {}

    @classmethod
    def from_workload(cls, w, T=None):
        return cls(w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T if T is None else T, w.k_bits, w.v_bits,
                   w.n_recent, w.log_window, getattr(w, "v_group", 32), getattr(w, "k_group", 32),
                   getattr(w, "key_rotation", False))

    def cache_sizes(self):
        arr = (ctypes.c_size_t * L_.KVQ_NUM_CACHE_BUFFERS)()
        L_.check(L_.load().kvq_cache_sizes(self.ref, arr))
        return dict(zip(L_.CACHE_FIELDS, list(arr)))

    def retained_positions(self):
        n = max(1, self.R)
        arr = (ctypes.c_int32 * n)()
        L_.check(L_.load().kvq_retained_positions(self.ref, arr, n))
        return list(arr)[: self.R]

    def quantized_before(self, t: int) -> int:
        return int(L_.load().kvq_quantized_before(self.ref, t))

    def workspace_bytes(self, num_partitions: int) -> int:
        n = self._ws.get(num_partitions)
        if n is None:
            n = self._ws[num_partitions] = int(L_.load().kvq_decode_workspace_bytes(self.ref, num_partitions))
        return n

    def shapes(self):
        """Tensor shape and dtype of each cache buffer (codes as int32 bit patterns)."""
        B, H, Tq, nG, R = self.B, self.Hkv, self.Tq, self.n_groups, self.R
        return {
            "k_codes": ((B, H, Tq, self.Dk * self.k_bits // 32), torch.int32),
            "k_scale": ((B, H, Tq // self.k_group, self.Dk), torch.float16),
            "k_zero": ((B, H, Tq // self.k_group, self.Dk), torch.float16),
            "v_codes": ((B, H, nG, self.Dv * self.v_bits), torch.int32),
            "v_scale": ((B, H, nG, self.Dv // self.v_group, 32), torch.float16),
            "v_zero": ((B, H, nG, self.Dv // self.v_group, 32), torch.float16),
            "k_fp16": ((B, H, R, self.Dk), torch.float16),
            "v_fp16": ((B, H, R, self.Dv), torch.float16),
        }


def decode_plan(layout: Layout, num_partitions: int, side_code: bool = False) -> dict:
    """Which decode kernel a request runs on the current device and how it is cut
    (kvq_decode_plan): kernel "mfma" or "valu", partial rows per query head, the
    matrix-core kernel's LDS ring depth and waves per SIMD, and the waves launched."""
    info = L_.KvqDecodeInfo()
    L_.check(L_.load().kvq_decode_plan(layout.ref, num_partitions, 1 if side_code else 0, ctypes.byref(info)))
    return {"kernel": {L_.KVQ_KERNEL_MFMA: "mfma", L_.KVQ_KERNEL_VALU: "valu"}[info.kernel], "units": info.units,
            "ring_depth": info.ring_depth, "waves_per_simd": info.waves_per_simd, "waves": info.waves}


def alloc_workspace(layout: Layout, num_partitions: int, device="cuda"):
    """Decode workspace for num_partitions partitions (needs no initialisation)."""
    need = layout.workspace_bytes(num_partitions)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def alloc_cache(layout: Layout, device="cuda"):
    """Caller-owned cache buffers (uninitialised) for a layout."""
    return {k: torch.empty(shape, dtype=dt, device=device) for k, (shape, dt) in layout.shapes().items()}


def _bind_cache(holder, shapes_fn, cache, allow_missing=True):
    """The kvq_cache struct of `cache` for a layout or stream `holder`.  It is built
    and checked once per set of tensor objects and reused while the same tensors
    are passed again (a decode loop passes the same cache every step); replacing a
    tensor's storage in place (``set_``) is not noticed."""
    tensors = tuple(cache.get(k) for k in L_.CACHE_FIELDS)
    memo = holder.__dict__.get("_cache_memo")
    if memo is not None and all(a is b for a, b in zip(memo[0], tensors)):
        return memo[1]
    c = L_.KvqCache()
    for k, (shape, dt) in shapes_fn().items():
        t = cache.get(k)
        if t is None:
            if not allow_missing:
                raise ValueError("cache[%r] is missing" % k)
            setattr(c, k, None)
            continue
        if tuple(t.shape) != tuple(shape) or t.dtype != dt or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("cache[%r] must be a contiguous CUDA %s tensor of shape %s" % (k, dt, shape))
        setattr(c, k, t.data_ptr() if t.numel() else None)
    holder.__dict__["_cache_memo"] = (tensors, c)
    return c


def _cache_struct(layout: Layout, cache):
    return _bind_cache(layout, layout.shapes, cache)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, t=None):
    """The HIP stream to enqueue on: `stream`, else the current stream of the device
    tensor t lives on (read without building a Stream object: a decode loop asks
    once per call), else of the current device."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if t is not None and _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(t.get_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_tensor(name, t, shape):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("%s must be a contiguous CUDA tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype not in _DTYPE_CODES:
        raise ValueError("%s dtype %s not supported (float32, float16, bfloat16)" % (name, t.dtype))


def kv_quant_pack(layout: Layout, K, V, cache=None, t_begin: int = 0, stream=None):
    """Quantize and pack positions [t_begin, t_begin + K.shape[2]) into ``cache``
    (allocated if None).  K [B, Hkv, t, Dk], V [B, Hkv, t, Dv] on the GPU."""
    t_count = K.shape[2]
    _check_tensor("K", K, (layout.B, layout.Hkv, t_count, layout.Dk))
    _check_tensor("V", V, (layout.B, layout.Hkv, t_count, layout.Dv))
    if K.dtype != V.dtype:
        raise ValueError("K and V must share a dtype")
    if cache is None:
        cache = alloc_cache(layout, K.device)
    cs = _cache_struct(layout, cache)
    L_.check(L_.load().kv_quant_pack(layout.ref, t_begin, t_count, ctypes.c_void_p(K.data_ptr()),
                                     ctypes.c_void_p(V.data_ptr()), _DTYPE_CODES[K.dtype], ctypes.byref(cs),
                                     _stream(stream, K)))
    return cache


def kv_decode_attn(layout: Layout, q, cache, num_partitions: int = 1, softmax_scale=None, out=None,
                   workspace=None, stream=None, after_decode_event=None, kernel_events=None):
    """Decode attention of q [B, Hq, Dk] over a packed cache -> float32 [B, Hq, Dv].

    after_decode_event: optional torch.cuda.Event, recorded on the stream between
    the decode kernel and the merge kernel (C ABI kv_decode_attn_ex).
    kernel_events: optional pair of torch.cuda.Event (start, stop), the start and
    stop events of the decode kernel's launch (C ABI kv_decode_attn_timed);
    not together with after_decode_event.  Events must have been recorded once
    before, so that torch has created them."""
    _check_tensor("q", q, (layout.B, layout.Hq, layout.Dk))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(layout.Dk)
    if out is None:
        out = torch.empty((layout.B, layout.Hq, layout.Dv), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (layout.B, layout.Hq, layout.Dv) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor [B, Hq, Dv]")
    need = layout.workspace_bytes(num_partitions)
    if need and workspace is None:
        workspace = alloc_workspace(layout, num_partitions, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    cs = _cache_struct(layout, cache)
    if kernel_events is not None:
        if after_decode_event is not None:
            raise ValueError("kernel_events and after_decode_event are exclusive")
        k0, k1 = (e.cuda_event for e in kernel_events)
        if not k0 or not k1:
            raise ValueError("kernel_events have not been created yet (record them once first)")
        L_.check(L_.load().kv_decode_attn_timed(layout.ref, ctypes.c_void_p(q.data_ptr()), _DTYPE_CODES[q.dtype],
                                                ctypes.byref(cs), ctypes.c_float(softmax_scale), num_partitions,
                                                ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.c_void_p(out.data_ptr()),
                                                _stream(stream, q), ctypes.c_void_p(k0), ctypes.c_void_p(k1)))
        return out
    ev = None
    if after_decode_event is not None:
        ev = after_decode_event.cuda_event
        if not ev:
            raise ValueError("after_decode_event has not been created yet (record it once first)")
    L_.check(L_.load().kv_decode_attn_ex(layout.ref, ctypes.c_void_p(q.data_ptr()), _DTYPE_CODES[q.dtype],
                                         ctypes.byref(cs), ctypes.c_float(softmax_scale), num_partitions,
                                         ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.c_void_p(out.data_ptr()),
                                         _stream(stream, q), ctypes.c_void_p(ev)))
    return out


def kv_decode_attn_noalloc(layout: Layout, q, cache, num_partitions: int = 1, softmax_scale=None, out=None,
                           stream=None):
    """kv_decode_attn without a workspace (C ABI kv_decode_attn_noalloc): the partial
    results go to the library's static per-GPU scratch, so the call allocates no
    device memory when ``out`` is given.  Calls that overlap on one GPU race."""
    _check_tensor("q", q, (layout.B, layout.Hq, layout.Dk))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(layout.Dk)
    if out is None:
        out = torch.empty((layout.B, layout.Hq, layout.Dv), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (layout.B, layout.Hq, layout.Dv) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor [B, Hq, Dv]")
    cs = _cache_struct(layout, cache)
    L_.check(L_.load().kv_decode_attn_noalloc(layout.ref, ctypes.c_void_p(q.data_ptr()), _DTYPE_CODES[q.dtype],
                                              ctypes.byref(cs), ctypes.c_float(softmax_scale), num_partitions,
                                              ctypes.c_void_p(out.data_ptr()), _stream(stream, q)))
    return out


def kvq_read_probe(buf, sink=None, stream=None):
    """Measurement support: read the bytes of the contiguous device tensor ``buf``
    once with a plain streaming read (C ABI kvq_read_probe), so that the caller can
    time the device's achievable HBM read rate.  ``sink``: a 4-byte device tensor
    the kernel may write (allocated if None)."""
    import torch
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=buf.device)
    L_.check(L_.load().kvq_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                      ctypes.c_void_p(sink.data_ptr()), _stream(stream, buf)))
    return sink


class Stream:
    """A streaming cache (kvq_stream of include/kvq.h): the host state and, unless
    device is None, its caller-owned device buffers (``cache``).  Tokens are
    appended one at a time (``append``); ``prefill`` starts an empty stream from
    the one-shot cache of its first tokens."""

    def __init__(self, B, Hq, Hkv, Dk, Dv, capacity, k_bits, v_bits, n_recent=0, log_window=0, device="cuda",
                 v_group=32, key_rotation=False):
        self._c = L_.KvqStream()
        lib = L_.load()
        L_.check(lib.kvq_stream_init_ex(ctypes.byref(self._c), B, Hq, Hkv, Dk, Dv, capacity, k_bits, v_bits,
                                        n_recent, log_window, v_group))
        if key_rotation:
            L_.check(lib.kvq_stream_set_flags(ctypes.byref(self._c), L_.KVQ_KEY_ROTATION))
        self.cache = None
        if device is not None:
            # read-only view: the buffers are the stream's for its whole life, so the
            # kvq_cache struct is built once (a new mapping assigned to `cache` is
            # bound again)
            self.cache = types.MappingProxyType(
                {k: torch.empty(shape, dtype=dt, device=device) for k, (shape, dt) in self.shapes().items()})
        self._lib = lib
        self._ref = ctypes.byref(self._c)
        self._ws = {}
        # the format fields never change: plain attributes (the stream's state fields
        # t, n_groups, ... are read from the struct on every access)
        self.__dict__.update({f: getattr(self._c.L, f) for f in ("B", "Hq", "Hkv", "Dk", "Dv", "k_bits", "v_bits",
                                                                  "n_recent", "log_window", "k_group", "v_group")})
        self._kshape = torch.Size((B, Hkv, Dk))
        self._vshape = torch.Size((B, Hkv, Dv))

    def __getattr__(self, name):
        if name in L_.STREAM_FIELDS:
            return getattr(self._c, name)
        if name in L_.LAYOUT_FIELDS:
            return getattr(self._c.L, name)
        raise AttributeError(name)

    @property
    def capacity(self):
        return self._c.L.T

    @property
    def ref(self):
        return ctypes.byref(self._c)

    def shapes(self):
        """Shape and dtype of each buffer (capacities g_cap groups, r_cap rows per slab)."""
        c = self._c
        B, H, G, R, Dk, Dv = c.L.B, c.L.Hkv, c.g_cap, c.r_cap, c.L.Dk, c.L.Dv
        return {
            "k_codes": ((B, H, G * 32, Dk * c.L.k_bits // 32), torch.int32),
            "k_scale": ((B, H, G, Dk), torch.float16),
            "k_zero": ((B, H, G, Dk), torch.float16),
            "v_codes": ((B, H, G, Dv * c.L.v_bits), torch.int32),
            "v_scale": ((B, H, G, Dv // c.L.v_group, 32), torch.float16),
            "v_zero": ((B, H, G, Dv // c.L.v_group, 32), torch.float16),
            "k_fp16": ((B, H, R, Dk), torch.float16),
            "v_fp16": ((B, H, R, Dv), torch.float16),
        }

    def cache_sizes(self):
        arr = (ctypes.c_size_t * L_.KVQ_NUM_CACHE_BUFFERS)()
        L_.check(L_.load().kvq_stream_cache_sizes(self.ref, arr))
        return dict(zip(L_.CACHE_FIELDS, list(arr)))

    def workspace_bytes(self, num_partitions: int) -> int:
        n = self._ws.get(num_partitions)
        if n is None:
            n = self._ws[num_partitions] = int(L_.load().kvq_stream_workspace_bytes(self.ref, num_partitions))
        return n

    def row_positions(self):
        """Position of the token held by each fp16 row in use."""
        return list(self._c.row_pos[: self._c.n_rows])

    def pending_rows(self):
        return [i for i in range(self._c.n_rows) if self._c.row_pending[i]]

    def plan(self):
        """Host bookkeeping of one append without any GPU work (kvq_stream_plan):
        advances the state by one token and returns what the device would do."""
        st = L_.KvqStreamStep()
        L_.check(L_.load().kvq_stream_plan(self.ref, ctypes.byref(st)))
        return {"new_row": st.new_row, "group": st.group, "member_rows": list(st.member_rows),
                "member_pos": list(st.member_pos), "moves": list(zip(st.move_src[: st.n_moves], st.move_dst[: st.n_moves]))}

    def _cache_struct(self):
        if self.cache is None:
            raise ValueError("this stream has no device buffers (created with device=None)")
        return _bind_cache(self, self.shapes, self.cache, allow_missing=False)

    def _cache_ref(self):
        """byref of the bound kvq_cache struct, rebuilt only when `cache` is replaced."""
        bound = self.__dict__.get("_bound")
        if bound is None or bound[0] is not self.cache:
            bound = (self.cache, ctypes.byref(self._cache_struct()))
            self.__dict__["_bound"] = bound
        return bound[1]

    def prefill(self, K, V, stream=None):
        """Start the (empty) stream from K [B, Hkv, T0, Dk], V [B, Hkv, T0, Dv]."""
        T0 = K.shape[2]
        _check_tensor("K", K, (self.B, self.Hkv, T0, self.Dk))
        _check_tensor("V", V, (self.B, self.Hkv, T0, self.Dv))
        if K.dtype != V.dtype:
            raise ValueError("K and V must share a dtype")
        cs = self._cache_struct()
        L_.check(L_.load().kv_stream_prefill(self.ref, T0, ctypes.c_void_p(K.data_ptr()),
                                             ctypes.c_void_p(V.data_ptr()), _DTYPE_CODES[K.dtype], ctypes.byref(cs),
                                             _stream(stream, K)))

    def append(self, k, v, stream=None):
        """Append one token: k [B, Hkv, Dk], v [B, Hkv, Dv] on the GPU.  (Called once
        per decode step: the checks read as few attributes as possible.)"""
        code = _DTYPE_CODES.get(k.dtype)
        if (code is None or k.dtype != v.dtype or k.shape != self._kshape or v.shape != self._vshape
                or not (k.is_cuda and v.is_cuda and k.is_contiguous() and v.is_contiguous())):
            _check_tensor("k", k, tuple(self._kshape))
            _check_tensor("v", v, tuple(self._vshape))
            raise ValueError("k and v must share a dtype")
        L_.check(self._lib.kv_stream_append(self._ref, k.data_ptr(), v.data_ptr(), code, self._cache_ref(),
                                            _stream(stream, k)))

    def decode(self, q, num_partitions: int = 1, softmax_scale=None, out=None, workspace=None, stream=None):
        """Decode attention of q [B, Hq, Dk] over the stream's tokens -> float32 [B, Hq, Dv]."""
        _check_tensor("q", q, (self.B, self.Hq, self.Dk))
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.Dk)
        if out is None:
            out = torch.empty((self.B, self.Hq, self.Dv), dtype=torch.float32, device=q.device)
        elif out.dtype != torch.float32 or tuple(out.shape) != (self.B, self.Hq, self.Dv) or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor [B, Hq, Dv]")
        need = self.workspace_bytes(num_partitions)
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        L_.check(self._lib.kv_stream_decode(self._ref, q.data_ptr(), _DTYPE_CODES[q.dtype], self._cache_ref(),
                                            ctypes.c_float(softmax_scale), num_partitions, ws_ptr, ws_bytes,
                                            out.data_ptr(), _stream(stream, q)))
        return out


# ------------------------------------------------------------ HeadQ side code
def side_pack(layout: Layout, K, cache, U, side_bits: int = 8, stream=None):
    """HeadQ write path over a packed cache: side code of every quantized token.
    K: the [B, Hkv, T, Dk] keys the cache was packed from; U float32 [Hkv, Dk, r].
    Returns (codes uint8 [B, Hkv, Tq, r], scale, zero int16 fp16 bits [B, Hkv, Tq])."""
    _check_tensor("K", K, (layout.B, layout.Hkv, layout.T, layout.Dk))
    if U.dtype != torch.float32 or not U.is_cuda or not U.is_contiguous() or U.dim() != 3 \
            or tuple(U.shape[:2]) != (layout.Hkv, layout.Dk):
        raise ValueError("U must be a contiguous float32 CUDA tensor [Hkv, Dk, r]")
    r = U.shape[2]
    Tq = layout.Tq
    codes = torch.empty((layout.B, layout.Hkv, Tq, r), dtype=torch.uint8, device=K.device)
    scale = torch.empty((layout.B, layout.Hkv, Tq), dtype=torch.int16, device=K.device)
    zero = torch.empty_like(scale)
    side = L_.KvqSide(codes.data_ptr(), scale.data_ptr(), zero.data_ptr())
    cs = _cache_struct(layout, cache)
    L_.check(L_.load().kv_side_pack(layout.ref, r, side_bits, ctypes.c_void_p(U.data_ptr()),
                                    ctypes.c_void_p(K.data_ptr()), _DTYPE_CODES[K.dtype], ctypes.byref(cs),
                                    ctypes.byref(side), _stream(stream, K)))
    return codes, scale, zero


def kv_decode_attn_side(layout: Layout, q, cache, U, side, num_partitions: int = 1, softmax_scale=None,
                        stream=None):
    """kv_decode_attn with the HeadQ logit correction of ``side`` (from side_pack)."""
    _check_tensor("q", q, (layout.B, layout.Hq, layout.Dk))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(layout.Dk)
    out = torch.empty((layout.B, layout.Hq, layout.Dv), dtype=torch.float32, device=q.device)
    need = layout.workspace_bytes(num_partitions)
    workspace = alloc_workspace(layout, num_partitions, q.device) if need else None
    codes, scale, zero = side
    sd = L_.KvqSide(codes.data_ptr(), scale.data_ptr(), zero.data_ptr())
    cs = _cache_struct(layout, cache)
    L_.check(L_.load().kv_decode_attn_side(
        layout.ref, ctypes.c_void_p(q.data_ptr()), _DTYPE_CODES[q.dtype], ctypes.byref(cs), U.shape[2],
        ctypes.c_void_p(U.data_ptr()), ctypes.byref(sd), ctypes.c_float(softmax_scale), num_partitions,
        ctypes.c_void_p(workspace.data_ptr() if workspace is not None else None),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        ctypes.c_void_p(out.data_ptr()), _stream(stream, q)))
    return out
