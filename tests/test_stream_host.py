"""Host bookkeeping of the streaming cache (C ABI kvq_stream_plan), CPU only.

The library's planner and the oracle's ``SlabStream`` are run side by side over
the same token sequence and must agree after every step on which positions sit in
fp16 rows, which of them are pending, and the members of every group.  No GPU
work: ``kvq_stream_plan`` only advances the host state.
"""

import numpy as np
import pytest

from oracle.kvq_stream import SlabStream

q = pytest.importorskip("quantized_decode_attention_kv_amd")
from quantized_decode_attention_kv_amd import _lib as L_  # noqa: E402


@pytest.mark.parametrize("n_recent,W,T", [(4, 4, 700), (16, 8, 900), (0, 0, 200), (7, 0, 400), (1, 1, 1100),
                                          (128, 128, 1500), (40, 16, 800)])
def test_planner_matches_oracle(n_recent, W, T):
    s = q.Stream(1, 4, 1, 32, 32, T + 5, 4, 2, n_recent=n_recent, log_window=W, device=None)
    o = SlabStream(32, 32, 4, 2, n_recent, W)
    zeros = np.zeros(32, dtype=np.float32)
    for t in range(T):
        step = s.plan()
        n_before = len(o.groups)
        o.append(zeros, zeros, "f32")
        rows = s.row_positions()
        assert step["new_row"] >= 0
        assert len(rows) == s.n_rows == len(o.rows)
        assert sorted(rows) == sorted(o.rows)
        assert sorted(rows[i] for i in s.pending_rows()) == sorted(o.pending)
        assert s.n_pending == len(o.pending) and s.n_groups == len(o.groups) and s.t == o.t
        if len(o.groups) > n_before:
            assert step["group"] == n_before
            assert step["member_pos"] == [int(p) for p in o.groups[-1]["pos"]]
            # the moves fill exactly the freed rows below the new end
            freed = {r for r in step["member_rows"] if r < s.n_rows}
            assert {d for _, d in step["moves"]} == freed
            assert all(src >= s.n_rows for src, _ in step["moves"])
        else:
            assert step["group"] == -1 and not step["moves"]


def test_planner_errors():
    with pytest.raises(q.KvqError) as e:
        q.Stream(1, 4, 1, 32, 32, 100, 4, 2, n_recent=2, log_window=4, device=None)
    assert e.value.status == L_.KVQ_ERR_UNSUPPORTED
    with pytest.raises(q.KvqError) as e:
        q.Stream(1, 4, 1, 32, 32, 100000, 4, 2, n_recent=5000, log_window=0, device=None)
    assert e.value.status == L_.KVQ_ERR_UNSUPPORTED   # more fp16 rows than the state can track
    with pytest.raises(q.KvqError) as e:
        q.Stream(1, 4, 1, 32, 32, 100, 5, 2, n_recent=4, device=None)
    assert e.value.status == L_.KVQ_ERR_UNSUPPORTED
    s = q.Stream(1, 4, 1, 32, 32, 3, 4, 2, n_recent=3, device=None)
    for _ in range(3):
        s.plan()
    with pytest.raises(q.KvqError) as e:
        s.plan()
    assert e.value.status == L_.KVQ_ERR_INVALID
    assert s.t == 3   # a failed call leaves the state as it was


def test_stream_sizes_and_capacities():
    s = q.Stream(2, 8, 2, 64, 128, 4096 + 7, 4, 2, n_recent=128, log_window=0, device=None)
    assert s.g_cap == (4096 + 7) // 32 and s.r_cap == 128 + 32
    sizes = s.cache_sizes()
    slabs = 4
    assert sizes["k_codes"] == slabs * s.g_cap * 32 * 64 * 4 // 32 * 4
    assert sizes["v_codes"] == slabs * s.g_cap * 128 * 2 * 4
    assert sizes["k_fp16"] == slabs * s.r_cap * 64 * 2
    for k, (shape, dt) in s.shapes().items():
        assert int(np.prod(shape)) * (4 if "codes" in k else 2) == sizes[k], k
    assert s.workspace_bytes(1) == 0 and s.workspace_bytes(4) == 2 * 8 * 4 * 8 * (128 + 4) * 4


def test_row_bound_holds_over_a_long_stream():
    """n_rows never exceeds r_cap (the planner also checks it) over a long stream
    with log-spaced retention, and the bound is not loose by much."""
    T = 20000
    s = q.Stream(1, 4, 1, 32, 32, T, 2, 2, n_recent=64, log_window=64, device=None)
    most = 0
    for _ in range(T):
        s.plan()
        most = max(most, s.n_rows)
    assert most <= s.r_cap <= most + 64
