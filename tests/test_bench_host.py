"""Host logic of bench.py (CPU only): byte accounting, the one-GPU guard and the
traffic lookup.

* The algorithmic bytes of the 128K and 32K decode and of the 128K prefill pack
  are the figures the workload definitions state (538,542,080 / 874,250,240 /
  169,345,024 bytes).
* Decode bytes equal the C library's own buffer sizes (kvq_cache_sizes, a host
  call) plus queries and output, for every format variant the bench times.
"""

import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import workload  # noqa: E402


def test_stated_byte_counts():
    w = workload("long_128k")
    assert bench.decode_bytes(w, 128, w.T - 128) == 538_542_080
    w32 = workload("logquant_32k")
    assert bench.decode_bytes(w32, 640, w32.T - 640) == 874_250_240
    # prefill chunk of 8192 tokens, 128 of them in the fp16 window
    assert bench.pack_bytes(w, 8192, 8192 - 128) == 169_345_024


@pytest.mark.parametrize("kg,vg", bench.FORMAT_VARIANTS)
def test_decode_bytes_match_library_sizes(kg, vg):
    from quantized_decode_attention_kv_amd import _lib as L_
    lib = L_.load()
    w = workload("long_128k").with_(k_group=kg, v_group=vg)
    lay = L_.KvqLayout()
    assert lib.kvq_layout_init_ex(ctypes.byref(lay), w.B, w.Hq, w.Hkv, w.Dk, w.Dv, w.T, w.k_bits, w.v_bits,
                                  w.n_recent, w.log_window, kg, vg) == 0
    sizes = (ctypes.c_size_t * 8)()
    assert lib.kvq_cache_sizes(ctypes.byref(lay), sizes) == 0
    q_out = w.B * w.Hq * w.Dk * 2 + w.B * w.Hq * w.Dv * 4
    assert bench.decode_bytes(w, lay.R, lay.Tq) == sum(sizes) + q_out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_matches_current_sources():
    t = bench.read_traffic()
    assert t is None or t > 500e6
    with open(bench.TRAFFIC_FILE) as f:
        text = f.read()
    if ("kernel_source_sha256_16: %s" % bench.kernel_source_hash()) not in text:
        assert t is None   # a summary of other sources is never reported
        pytest.skip("the committed traffic summary predates the current decode sources")
    assert t is not None
