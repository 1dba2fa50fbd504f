"""Host-side tests of the C-ABI library (no GPU needed).

The library loads, exports every entry point include/kvq.h declares, derives the
same retained / quantized token sets as the oracle, reports buffer sizes that match
the oracle's packed arrays, and rejects invalid requests before launching anything.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from quantized_decode_attention_kv_amd import _lib as L_
from workloads import WORKLOADS, small_cases

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L_.LIB_PATH):
        from quantized_decode_attention_kv_amd import build
        build.build()
    return L_.load()


def _layout(lib, *args):
    lay = L_.KvqLayout()
    st = lib.kvq_layout_init(ctypes.byref(lay), *args)
    return st, lay


def test_header_symbols_exported(lib):
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(kvq?_\w+)\s*\(", text, flags=re.M))
    assert names == set(L_.EXPORTS), names ^ set(L_.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_library_does_not_reference_oracle():
    srcdir = os.path.join(ROOT, "quantized_decode_attention_kv_amd")
    for dirpath, _, files in os.walk(srcdir):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                body = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in body.replace("the oracle", ""), f


@pytest.mark.parametrize("w", WORKLOADS + small_cases(), ids=lambda w: w.name)
def test_layout_matches_oracle_retention(lib, w):
    st, lay = _layout(lib, w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T, w.k_bits, w.v_bits, w.n_recent, w.log_window)
    assert st == 0, lib.kvq_last_error()
    r, u = O.split_positions(w.T, w.n_recent, w.log_window)
    assert (lay.R, lay.Tq, lay.n_groups) == (len(r), len(u), len(u) // 32)
    if w.T <= 40000:
        arr = (ctypes.c_int32 * max(1, lay.R))()
        assert lib.kvq_retained_positions(ctypes.byref(lay), arr, max(1, lay.R)) == 0
        assert list(arr)[: lay.R] == r.tolist()
    # quantized_before at a few cut points
    for t in [0, 1, w.T // 3, w.T - 129, w.T - 1, w.T]:
        t = max(0, min(w.T, t))
        assert lib.kvq_quantized_before(ctypes.byref(lay), t) == int(np.sum(u < t))


@pytest.mark.parametrize("T,n_recent,W", [(777, 50, 32), (579, 0, 32), (1000, 8, 16), (4096, 128, 0), (96, 96, 0),
                                          (131072, 128, 0), (2048, 64, 64)])
def test_retention_host_vs_oracle(lib, T, n_recent, W):
    r, u = O.split_positions(T, n_recent, W)
    lay = L_.KvqLayout(B=1, Hq=1, Hkv=1, Dk=32, Dv=32, T=T, k_bits=4, v_bits=2, n_recent=n_recent, log_window=W,
                       k_group=32, v_group=32, R=len(r), Tq=len(u), n_groups=len(u) // 32)
    if len(u) % 32:
        # layouts with a partial group are refused; the counting itself is checked via init's message
        st, _ = _layout(lib, 1, 1, 1, 32, 32, T, 4, 2, n_recent, W)
        assert st == L_.KVQ_ERR_UNSUPPORTED
        return
    arr = (ctypes.c_int32 * max(1, len(r)))()
    assert lib.kvq_retained_positions(ctypes.byref(lay), arr, max(1, len(r))) == 0
    assert list(arr)[: len(r)] == r.tolist()


def test_cache_sizes_match_oracle_arrays(lib):
    for w in small_cases():
        lay = L_.KvqLayout()
        st = lib.kvq_layout_init_ex(ctypes.byref(lay), w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T, w.k_bits, w.v_bits,
                                    w.n_recent, w.log_window, w.k_group, w.v_group)
        assert st == 0
        sizes = (ctypes.c_size_t * 8)()
        assert lib.kvq_cache_sizes(ctypes.byref(lay), sizes) == 0
        from workloads import make_all
        K, V = make_all(w.with_(B=1, Hkv=1, Hq=w.G), workers=1)
        p = O.pack_slab(K[0, 0], V[0, 0], w.dtype, w.k_bits, w.v_bits, w.n_recent, w.log_window, v_group=w.v_group,
                        k_group=w.k_group)
        for i, k in enumerate(O.CACHE_KEYS):
            assert sizes[i] == p[k].nbytes * w.B * w.Hkv, k


@pytest.mark.parametrize("args,status", [
    ((1, 4, 2, 128, 128, 256, 3, 2, 0, 0), L_.KVQ_OK),                # 3-bit keys (bit streams)
    ((1, 4, 2, 128, 128, 256, 4, 3, 0, 0), L_.KVQ_OK),                # 3-bit values
    ((1, 4, 2, 128, 128, 256, 5, 2, 0, 0), L_.KVQ_ERR_UNSUPPORTED),   # 5-bit keys
    ((1, 4, 2, 128, 128, 256, 4, 6, 0, 0), L_.KVQ_ERR_UNSUPPORTED),   # 6-bit values
    ((1, 5, 2, 128, 128, 256, 4, 2, 0, 0), L_.KVQ_ERR_INVALID),       # Hq % Hkv
    ((1, 6, 2, 128, 128, 256, 4, 2, 0, 0), L_.KVQ_ERR_UNSUPPORTED),   # group of 3 queries
    ((1, 4, 2, 100, 128, 256, 4, 2, 0, 0), L_.KVQ_ERR_INVALID),       # Dk not a multiple of 32
    ((1, 4, 2, 512, 128, 256, 4, 2, 0, 0), L_.KVQ_ERR_UNSUPPORTED),   # Dk too wide
    ((1, 4, 2, 128, 128, 250, 4, 2, 0, 0), L_.KVQ_ERR_UNSUPPORTED),   # Tq % 32
    ((1, 4, 2, 128, 128, 256, 4, 2, 300, 0), L_.KVQ_ERR_INVALID),     # n_recent > T
    ((0, 4, 2, 128, 128, 256, 4, 2, 0, 0), L_.KVQ_ERR_INVALID),       # B = 0
    ((1, 4, 2, 128, 128, 256, 4, 2, 0, -1), L_.KVQ_ERR_INVALID),      # negative window
])
def test_layout_errors(lib, args, status):
    st, _ = _layout(lib, *args)
    assert st == status
    if status != L_.KVQ_OK:
        assert lib.kvq_last_error().decode()


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced: every call below fails validation


def _cache(ptr=FAKE):
    return L_.KvqCache(*([ptr] * 8))


def test_pack_errors(lib):
    st, lay = _layout(lib, 1, 4, 2, 128, 128, 320, 4, 2, 64, 0)   # R = 64, Tq = 256
    assert st == 0
    ok_cache = _cache()
    pack = lambda t0, tc, K=FAKE, V=FAKE, dt=L_.KVQ_BF16, cache=ok_cache: lib.kv_quant_pack(
        ctypes.byref(lay), t0, tc, K, V, dt, ctypes.byref(cache) if cache is not None else None, None)
    assert pack(0, 320, K=None) == L_.KVQ_ERR_INVALID
    assert pack(0, 320, K=FAKE + 2) == L_.KVQ_ERR_INVALID          # misaligned
    assert pack(0, 320, dt=7) == L_.KVQ_ERR_INVALID
    assert pack(0, 321) == L_.KVQ_ERR_INVALID                      # past T
    assert pack(-1, 10) == L_.KVQ_ERR_INVALID
    assert pack(0, 0) == L_.KVQ_ERR_INVALID
    assert pack(0, 100) == L_.KVQ_ERR_UNSUPPORTED                  # splits a key group
    assert pack(0, 320, cache=None) == L_.KVQ_ERR_INVALID
    bad = _cache()
    bad.k_zero = None
    assert pack(0, 320, cache=bad) == L_.KVQ_ERR_INVALID
    bad = _cache()
    bad.v_fp16 = FAKE + 4
    assert pack(0, 320, cache=bad) == L_.KVQ_ERR_INVALID
    stale = L_.KvqLayout.from_buffer_copy(lay)
    stale.R = 0
    assert lib.kv_quant_pack(ctypes.byref(stale), 0, 320, FAKE, FAKE, L_.KVQ_BF16, ctypes.byref(ok_cache),
                             None) == L_.KVQ_ERR_INVALID


def test_decode_errors(lib):
    st, lay = _layout(lib, 2, 8, 2, 128, 128, 1088, 4, 2, 64, 0)   # 32 groups, R = 64
    assert st == 0
    need = lib.kvq_decode_workspace_bytes(ctypes.byref(lay), 4)
    assert need == 2 * 8 * 8 * 4 * 132 * 4            # B * Hq * 8P * (Dv + 4) floats of partials
    assert lib.kvq_decode_workspace_bytes(ctypes.byref(lay), 1) == 0
    c = _cache()
    dec = lambda q=FAKE, qd=L_.KVQ_BF16, sc=0.1, P=4, ws=FAKE, wsb=need, out=FAKE, cache=c: lib.kv_decode_attn(
        ctypes.byref(lay), q, qd, ctypes.byref(cache), ctypes.c_float(sc), P, ws, wsb, out, None)
    assert dec(q=None) == L_.KVQ_ERR_INVALID
    assert dec(out=None) == L_.KVQ_ERR_INVALID
    assert dec(out=FAKE + 8) == L_.KVQ_ERR_INVALID
    assert dec(qd=9) == L_.KVQ_ERR_INVALID
    assert dec(sc=float("nan")) == L_.KVQ_ERR_INVALID
    assert dec(sc=float("inf")) == L_.KVQ_ERR_INVALID
    assert dec(P=0) == L_.KVQ_ERR_INVALID
    assert dec(P=35) == L_.KVQ_ERR_INVALID                        # > ceil(T/32) = 34
    assert dec(ws=None) == L_.KVQ_ERR_INVALID
    assert dec(ws=FAKE + 4) == L_.KVQ_ERR_INVALID
    least = 2 * 8 * 4 * 132 * 4                                    # at least P partial rows per query head
    assert dec(wsb=least - 4) == L_.KVQ_ERR_INVALID
    bad = _cache()
    bad.k_fp16 = None
    assert dec(cache=bad) == L_.KVQ_ERR_INVALID
    bad = _cache()
    bad.v_codes = None
    assert dec(cache=bad) == L_.KVQ_ERR_INVALID
    # the timed entry point runs the same checks before any launch
    timed = lambda q=FAKE, P=4: lib.kv_decode_attn_timed(ctypes.byref(lay), q, L_.KVQ_BF16, ctypes.byref(c),
                                                         ctypes.c_float(0.1), P, FAKE, need, FAKE, None, None, None)
    assert timed(q=None) == L_.KVQ_ERR_INVALID
    assert timed(P=35) == L_.KVQ_ERR_INVALID


def test_read_probe_errors(lib):
    # argument checks happen on the host, before any launch
    assert lib.kvq_read_probe(None, 4096, FAKE, None) == L_.KVQ_ERR_INVALID
    assert lib.kvq_read_probe(FAKE, 4096, None, None) == L_.KVQ_ERR_INVALID
    assert lib.kvq_read_probe(FAKE + 8, 4096, FAKE, None) == L_.KVQ_ERR_INVALID
    assert lib.kvq_read_probe(FAKE, 4096, FAKE + 2, None) == L_.KVQ_ERR_INVALID


def test_status_strings(lib):
    for s in range(4):
        assert lib.kvq_status_string(s)
    assert b"unknown" in lib.kvq_status_string(42)


@pytest.mark.parametrize("Dv,vg,status", [(128, 48, L_.KVQ_ERR_UNSUPPORTED), (96, 64, L_.KVQ_ERR_UNSUPPORTED),
                                          (64, 128, L_.KVQ_ERR_UNSUPPORTED), (128, 128, L_.KVQ_OK),
                                          (192, 64, L_.KVQ_OK)])
def test_value_group_limits(lib, Dv, vg, status):
    lay = L_.KvqLayout()
    assert lib.kvq_layout_init_ex(ctypes.byref(lay), 1, 4, 2, 128, Dv, 256, 4, 2, 0, 0, 32, vg) == status
    if status == L_.KVQ_OK:
        sizes = (ctypes.c_size_t * 8)()
        assert lib.kvq_cache_sizes(ctypes.byref(lay), sizes) == 0
        assert sizes[4] == 2 * (256 // 32) * 32 * (Dv // vg) * 2   # v_scale: slabs x groups x Dv/vg x 32 fp16
    # the default init is value groups of 32
    assert lib.kvq_layout_init(ctypes.byref(lay), 1, 4, 2, 128, 128, 256, 4, 2, 0, 0) == 0 and lay.v_group == 32


@pytest.mark.parametrize("T,n_recent,kg,status", [(256, 0, 64, L_.KVQ_OK), (256, 0, 128, L_.KVQ_OK),
                                                  (288, 32, 128, L_.KVQ_OK), (288, 0, 128, L_.KVQ_ERR_UNSUPPORTED),
                                                  (256, 0, 96, L_.KVQ_ERR_UNSUPPORTED)])
def test_key_group_limits(lib, T, n_recent, kg, status):
    lay = L_.KvqLayout()
    assert lib.kvq_layout_init_ex(ctypes.byref(lay), 1, 4, 2, 128, 128, T, 4, 2, n_recent, 0, kg, 32) == status
    if status == L_.KVQ_OK:
        sizes = (ctypes.c_size_t * 8)()
        assert lib.kvq_cache_sizes(ctypes.byref(lay), sizes) == 0
        assert sizes[1] == 2 * (lay.Tq // kg) * 128 * 2     # k_scale: slabs x key groups x Dk fp16
        # a chunk must not split a key group
        assert lib.kv_quant_pack(ctypes.byref(lay), 0, 32, ctypes.c_void_p(16), ctypes.c_void_p(16), L_.KVQ_BF16,
                                 ctypes.byref(L_.KvqCache()), None) == L_.KVQ_ERR_UNSUPPORTED


def test_layout_and_stream_flags(lib):
    """Key rotation is a layout flag: set on a power-of-two key width, refused
    otherwise, unknown bits refused, the layout untouched by a refused call; side
    codes refuse a flagged layout; a stream takes flags only while empty."""
    st, lay = _layout(lib, 1, 4, 2, 128, 128, 256, 4, 2, 0, 0)
    assert st == L_.KVQ_OK and lay.flags == 0
    assert lib.kvq_layout_set_flags(ctypes.byref(lay), L_.KVQ_KEY_ROTATION) == L_.KVQ_OK
    assert lay.flags == L_.KVQ_KEY_ROTATION
    assert lib.kvq_layout_set_flags(ctypes.byref(lay), 2) == L_.KVQ_ERR_INVALID
    assert lay.flags == L_.KVQ_KEY_ROTATION
    st, lay96 = _layout(lib, 1, 4, 2, 96, 128, 256, 4, 2, 0, 0)
    assert lib.kvq_layout_set_flags(ctypes.byref(lay96), L_.KVQ_KEY_ROTATION) == L_.KVQ_ERR_UNSUPPORTED
    assert lay96.flags == 0
    bad = L_.KvqLayout.from_buffer_copy(lay)
    bad.flags = 4                                                  # set behind the library's back
    cache = _cache()
    assert lib.kv_quant_pack(ctypes.byref(bad), 0, 256, FAKE, FAKE, L_.KVQ_BF16, ctypes.byref(cache),
                             None) == L_.KVQ_ERR_INVALID
    side = L_.KvqSide(FAKE, FAKE, FAKE)
    assert lib.kv_side_pack(ctypes.byref(lay), 4, 4, FAKE, FAKE, L_.KVQ_BF16, ctypes.byref(cache),
                            ctypes.byref(side), None) == L_.KVQ_ERR_UNSUPPORTED
    S = L_.KvqStream()
    assert lib.kvq_stream_init(ctypes.byref(S), 1, 4, 1, 64, 64, 200, 4, 2, 8, 0) == L_.KVQ_OK
    assert lib.kvq_stream_set_flags(ctypes.byref(S), 8) == L_.KVQ_ERR_INVALID
    assert lib.kvq_stream_set_flags(ctypes.byref(S), L_.KVQ_KEY_ROTATION) == L_.KVQ_OK
    assert S.L.flags == L_.KVQ_KEY_ROTATION
    step = L_.KvqStreamStep()
    assert lib.kvq_stream_plan(ctypes.byref(S), ctypes.byref(step)) == L_.KVQ_OK
    assert lib.kvq_stream_set_flags(ctypes.byref(S), 0) == L_.KVQ_ERR_INVALID   # no longer empty
    assert S.L.flags == L_.KVQ_KEY_ROTATION
    S96 = L_.KvqStream()
    assert lib.kvq_stream_init(ctypes.byref(S96), 1, 4, 1, 96, 64, 200, 4, 2, 8, 0) == L_.KVQ_OK
    assert lib.kvq_stream_set_flags(ctypes.byref(S96), L_.KVQ_KEY_ROTATION) == L_.KVQ_ERR_UNSUPPORTED
