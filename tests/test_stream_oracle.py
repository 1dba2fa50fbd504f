"""Pins of the streaming-cache oracle (CPU only).

The oracle appends one token at a time (LogQuant technical summary, section 2,
dynamic adjustment; section 4, order-free attention).  It is pinned here against
facts that do not come from its own code:

* closed form of the step at which a position leaves the fp16 set: with window
  n_recent >= W = log_window > 0, position p (p = 2^v * odd) is retained while its
  distance d = t - p satisfies d <= max(n_recent, W * 2^v) (the span j holding
  W*2^(j-1) < d <= W*2^j keeps the multiples of 2^j, i.e. j <= v), so it leaves at
  t = p + max(n_recent, W * 2^v) + 1, and position 0 never leaves; with W = 0 it
  leaves at t = p + n_recent + 1;
* group formation replayed from those closed-form times alone: each group is the 32
  lowest-position tokens that have left the set and are not yet packed, formed at
  the step where the 32nd of them arrives;
* with W = 0 the tokens leave in position order, so the stream must equal the
  one-shot cache (``pack_slab``, pinned by the hand examples) bit for bit whenever
  its quantized count is a multiple of 32 and the inputs are exact in fp16;
* with every token retained, decode is plain softmax attention over the fp16-rounded
  keys and values (scipy's softmax).
"""

import numpy as np
import pytest
from scipy.special import softmax

from oracle import pack_slab, split_positions
from oracle.kvq_stream import SlabStream


def _v2(p: int) -> int:
    return (p & -p).bit_length() - 1


def _leave_step(p: int, n_recent: int, W: int):
    """Step count t at which position p first is not retained (None: never)."""
    if W == 0:
        return p + n_recent + 1
    if p == 0:
        return None
    return p + max(n_recent, W << _v2(p)) + 1


def _fp16_rows(rng, T, D):
    """fp16 bit patterns of N(0, 1) values: exact in fp16, so storing a token in fp16
    changes nothing and the stream can be compared with a one-shot pack bit for bit."""
    return rng.standard_normal((T, D)).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("n_recent,W", [(4, 4), (8, 4), (6, 2), (5, 0), (0, 0), (33, 0)])
def test_leave_steps_match_closed_form(n_recent, W):
    rng = np.random.default_rng(11)
    T = 700
    K, V = _fp16_rows(rng, T, 32), _fp16_rows(rng, T, 32)
    s = SlabStream(32, 32, 4, 2, n_recent, W)
    left_at = {}
    for t in range(T):
        s.append(K[t], V[t], "f16")
        fp16_set = set(s.rows) - s.pending
        for p in range(s.t):
            if p not in fp16_set and p not in left_at:
                left_at[p] = s.t
    for p in range(T):
        expect = _leave_step(p, n_recent, W)
        if expect is None or expect > T:
            assert p not in left_at, p
        else:
            assert left_at.get(p) == expect, (p, left_at.get(p), expect)


@pytest.mark.parametrize("n_recent,W,T", [(4, 4, 900), (16, 8, 900), (0, 0, 900), (7, 0, 900), (1, 1, 1100)])
def test_groups_replayed_from_closed_form(n_recent, W, T):
    """Conservation and group membership, replayed without the oracle's retention code.
    With n_recent = W = 1, m positions leave at once at t = 2^m + 1, so some groups
    are chosen from more than 32 waiting tokens (which of them is then decided by
    position, not by arrival)."""
    rng = np.random.default_rng(12)
    K, V = _fp16_rows(rng, T, 32), _fp16_rows(rng, T, 64)
    s = SlabStream(32, 64, 2, 4, n_recent, W)
    waiting, expected_groups, most_waiting = [], [], 0
    for t in range(T):
        s.append(K[t], V[t], "f16")
        # positions whose closed-form leave step is this step join the waiting list
        waiting += [p for p in range(s.t) if _leave_step(p, n_recent, W) == s.t]
        most_waiting = max(most_waiting, len(waiting))
        while len(waiting) >= 32:
            waiting.sort()
            expected_groups.append(waiting[:32])
            waiting = waiting[32:]
        assert len(s.pending) < 32
        assert sorted(s.pending) == sorted(waiting)
        grouped = [int(p) for g in s.groups for p in g["pos"]]
        assert sorted(grouped + list(s.rows)) == list(range(s.t))  # every token exactly once
    assert [list(g["pos"]) for g in s.groups] == expected_groups
    assert len(expected_groups) > 3
    if W == 1:
        assert most_waiting > 32


@pytest.mark.parametrize("kb,vb,n_recent", [(4, 2, 16), (2, 2, 0), (8, 4, 40), (3, 3, 8)])
def test_stream_equals_one_shot_without_log_window(kb, vb, n_recent):
    rng = np.random.default_rng(13)
    Dk, Dv = 64, 128
    T = n_recent + 32 * 6
    K, V = _fp16_rows(rng, T, Dk), _fp16_rows(rng, T, Dv)
    K[:, 3] = (rng.standard_normal(T) * 8 + 2).astype(np.float16).view(np.uint16)  # outlier channel
    s = SlabStream(Dk, Dv, kb, vb, n_recent, 0)
    for t in range(T):
        s.append(K[t], V[t], "f16")
        if (s.t - n_recent) % 32 == 0 and s.t >= n_recent:
            p, gpos, rpos = s.as_packed()
            ref = pack_slab(K[:s.t], V[:s.t], "f16", kb, vb, n_recent, 0)
            r, u = split_positions(s.t, n_recent, 0)
            assert np.array_equal(gpos, u) and np.array_equal(rpos, r)
            for key in ref:
                assert np.array_equal(p[key], ref[key]), (s.t, key)


def test_prefill_then_append_equals_one_shot():
    rng = np.random.default_rng(14)
    Dk, Dv, n_recent = 32, 64, 8
    T0, T1 = n_recent + 64, n_recent + 32 * 5
    K, V = _fp16_rows(rng, T1, Dk), _fp16_rows(rng, T1, Dv)
    s = SlabStream(Dk, Dv, 4, 2, n_recent, 0)
    s.prefill(K[:T0], V[:T0], "f16")
    for t in range(T0, T1):
        s.append(K[t], V[t], "f16")
    p, _, _ = s.as_packed()
    ref = pack_slab(K, V, "f16", 4, 2, n_recent, 0)
    for key in ref:
        assert np.array_equal(p[key], ref[key]), key


def test_groups_quantized_from_the_fp16_copies():
    """float32 inputs: the stream stores each token in fp16 first, so its groups equal
    the one-shot cache of the fp16-rounded inputs (and not of the float32 ones)."""
    rng = np.random.default_rng(16)
    Dk, Dv, n_recent = 32, 32, 4
    T = n_recent + 32 * 3
    K = (rng.standard_normal((T, Dk)) * 3).astype(np.float32)
    V = rng.standard_normal((T, Dv)).astype(np.float32)
    s = SlabStream(Dk, Dv, 4, 4, n_recent, 0)
    for t in range(T):
        s.append(K[t], V[t], "f32")
    p, _, _ = s.as_packed()
    ref16 = pack_slab(K.astype(np.float16).view(np.uint16), V.astype(np.float16).view(np.uint16),
                      "f16", 4, 4, n_recent, 0)
    ref32 = pack_slab(K, V, "f32", 4, 4, n_recent, 0)
    for key in ref16:
        assert np.array_equal(p[key], ref16[key]), key
    assert not np.array_equal(p["k_codes"], ref32["k_codes"])


def test_all_retained_decode_is_plain_attention():
    rng = np.random.default_rng(15)
    Dk, Dv, T, G = 64, 32, 50, 4
    K = rng.standard_normal((T, Dk)).astype(np.float32)
    V = rng.standard_normal((T, Dv)).astype(np.float32)
    q = rng.standard_normal((G, Dk)).astype(np.float32)
    s = SlabStream(Dk, Dv, 2, 2, T, 0)
    for t in range(T):
        s.append(K[t], V[t], "f32")
    assert not s.groups and len(s.rows) == T
    scale = 0.125
    K16 = K.astype(np.float16).astype(np.float64)
    V16 = V.astype(np.float16).astype(np.float64)
    ref = softmax(scale * (q.astype(np.float64) @ K16.T), axis=-1) @ V16
    assert np.allclose(s.decode(q, "f32", scale), ref, rtol=0, atol=1e-12)


def test_stream_rejects_reentering_window():
    with pytest.raises(ValueError):
        SlabStream(32, 32, 4, 2, 2, 4)


# ------------------------------------------------------------------ key rotation
# With key rotation ("Quantize What Counts", rotation integration) the stream stores
# each key rotated by the orthonormal Walsh-Hadamard transform (Sylvester order,
# scipy.linalg.hadamard) and decode rotates the query.

def _sylvester(n):
    from scipy.linalg import hadamard
    return hadamard(n).astype(np.float64)


def test_rotated_stream_equals_rotated_one_shot_without_log_window():
    """Keys built as H Y / 8 (Dk = 64) from integer multiples of 1/8: every step of the
    rotation is exact, so the rotated keys are Y, exact in fp16, and the rotated stream
    must equal the rotated one-shot cache bit for bit (the rotation comes before the
    fp16 copy, and groups form from the rotated rows)."""
    rng = np.random.default_rng(17)
    Dk, Dv, n_recent = 64, 64, 8
    T = n_recent + 32 * 4
    Y = rng.integers(-16, 17, size=(T, Dk)) / 8.0
    Y[:, 5] += 24.0                                           # an outlier channel after rotation
    K = (Y @ _sylvester(Dk).T / 8.0).astype(np.float32)       # exact: sums of multiples of 1/64
    V = rng.standard_normal((T, Dv)).astype(np.float16).view(np.uint16).view(np.float16).astype(np.float32)
    s = SlabStream(Dk, Dv, 4, 2, n_recent, 0, key_rotation=True)
    for t in range(T):
        s.append(K[t], V[t], "f32")
    p, _, _ = s.as_packed()
    ref = pack_slab(K, V, "f32", 4, 2, n_recent, 0, key_rotation=True)
    for key in ref:
        assert np.array_equal(p[key], ref[key]), key
    assert np.array_equal(p["k_fp16"].view(np.float16).astype(np.float64), Y[-n_recent:])
    plain = pack_slab(K, V, "f32", 4, 2, n_recent, 0)
    assert not np.array_equal(plain["k_codes"], ref["k_codes"])


def test_rotated_stream_all_retained_decode_keeps_scores():
    """Every token retained: the fp16 rows are fp16(H k / 8) (within one fp16 rounding of
    the float64 product) and decode with the rotated query is plain attention, since
    (H q) . (H k) / 64 = q . k: it matches scipy's softmax over the plain keys to the
    error of one fp16 rounding of each key."""
    rng = np.random.default_rng(18)
    Dk, Dv, T, G = 64, 32, 40, 4
    K = rng.standard_normal((T, Dk)).astype(np.float32)
    V = rng.standard_normal((T, Dv)).astype(np.float32)
    q = rng.standard_normal((G, Dk)).astype(np.float32)
    s = SlabStream(Dk, Dv, 2, 2, T, 0, key_rotation=True)
    for t in range(T):
        s.append(K[t], V[t], "f32")
    p, _, _ = s.as_packed()
    rot64 = K.astype(np.float64) @ _sylvester(Dk).T / 8.0
    got = p["k_fp16"].view(np.float16).astype(np.float64)
    assert np.all(np.abs(got - rot64) <= np.abs(rot64) * 2.0 ** -10 + 2.0 ** -24)
    scale = 0.125
    ref = softmax(scale * (q.astype(np.float64) @ K.astype(np.float64).T), axis=-1) @ V.astype(np.float16).astype(np.float64)
    assert np.abs(s.decode(q, "f32", scale) - ref).max() < 5e-3
