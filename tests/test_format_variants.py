"""Pins of the value-group width and the key-group length (CPU only).

"Quantize What Counts" (results) sweeps the quantization group size; the library
takes values in groups of v_group = 32, 64 or 128 channels per token.  The oracle's
grouping is pinned against:

* a closed form: with one group per row (v_group = Dv) each token's scale and zero
  are fp16((max - min) / (2^b - 1)) and fp16(min) of the whole row, computed here
  with numpy's row maximum and minimum;
* a reduction to the pinned 32-channel grouping: when the two 32-channel halves of
  every 64-channel group share their minimum and maximum, v_group = 64 must give
  the same codes as v_group = 32, and its scale / zero must equal both halves';
* dequantization through the scale array's width: the reconstruction of every value
  lies within half a step (plus the fp16 rounding of the zero) of the input.
"""

import numpy as np
import pytest

from oracle import dequant_slab, pack_slab, unpack_codes, unpack_value_codes


def _v_rows(rng, T, Dv):
    return (rng.standard_normal((T, Dv)) * 0.5).astype(np.float32)


@pytest.mark.parametrize("vb", [2, 3, 4, 8])
def test_whole_row_group_closed_form(vb):
    rng = np.random.default_rng(31)
    T, Dk, Dv = 64, 32, 128
    K = rng.standard_normal((T, Dk)).astype(np.float32)
    V = _v_rows(rng, T, Dv)
    p = pack_slab(K, V, "f32", 4, vb, 0, 0, v_group=Dv)
    assert p["v_scale"].shape == (2, 1, 32)
    s = p["v_scale"].view(np.float16)[:, 0, :].reshape(T)        # token 32 g + t
    z = p["v_zero"].view(np.float16)[:, 0, :].reshape(T)
    levels = np.float32(2 ** vb - 1)
    want_s = ((V.max(axis=1) - V.min(axis=1)) / levels).astype(np.float16)
    want_z = V.min(axis=1).astype(np.float16)
    assert np.array_equal(s.view(np.uint16), want_s.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), want_z.view(np.uint16))


@pytest.mark.parametrize("vb", [2, 4])
def test_64_group_reduces_to_32_when_halves_share_range(vb):
    rng = np.random.default_rng(32)
    T, Dk, Dv = 96, 32, 128
    K = rng.standard_normal((T, Dk)).astype(np.float32)
    V = _v_rows(rng, T, Dv)
    lo, hi = V.min(axis=1) - 1.0, V.max(axis=1) + 1.0
    for g0 in range(0, Dv, 64):          # both halves of every 64-group reach lo and hi
        for h0 in (g0, g0 + 32):
            V[:, h0 + 3] = lo
            V[:, h0 + 17] = hi
    p32 = pack_slab(K, V, "f32", 4, vb, 0, 0, v_group=32)
    p64 = pack_slab(K, V, "f32", 4, vb, 0, 0, v_group=64)
    assert np.array_equal(p32["v_codes"], p64["v_codes"])
    for key in ("v_scale", "v_zero"):
        a32, a64 = p32[key], p64[key]                              # [nG, 4, 32], [nG, 2, 32]
        assert np.array_equal(a32[:, 0::2], a64) and np.array_equal(a32[:, 1::2], a64)
    assert not np.array_equal(pack_slab(K, V + np.linspace(0, 1, Dv, dtype=np.float32), "f32", 4, vb, 0, 0,
                                        v_group=64)["v_scale"][:, 0], p64["v_scale"][:, 0])


@pytest.mark.parametrize("vg", [32, 64, 128])
def test_dequant_within_half_step(vg):
    rng = np.random.default_rng(33)
    T, Dk, Dv, vb = 64, 32, 128, 4
    K = rng.standard_normal((T, Dk)).astype(np.float32)
    V = _v_rows(rng, T, Dv)
    p = pack_slab(K, V, "f32", 4, vb, 0, 0, v_group=vg)
    _, Vhat = dequant_slab(p, 4, vb)
    s = np.repeat(p["v_scale"].view(np.float16).astype(np.float64).transpose(0, 2, 1).reshape(T, Dv // vg), vg, axis=1)
    z = np.repeat(p["v_zero"].view(np.float16).astype(np.float64).transpose(0, 2, 1).reshape(T, Dv // vg), vg, axis=1)
    mn = np.repeat(V.reshape(T, Dv // vg, vg).min(axis=2).astype(np.float64), vg, axis=1)
    err = np.abs(Vhat - V.astype(np.float64))
    assert np.all(err <= 0.5 * s + np.abs(z - mn) + 1e-6)
    codes = unpack_value_codes(p["v_codes"], vb)
    assert codes.max() <= 2 ** vb - 1


def test_bad_value_group():
    K = np.zeros((32, 32), np.float32)
    with pytest.raises(ValueError):
        pack_slab(K, np.zeros((32, 96), np.float32), "f32", 4, 2, 0, 0, v_group=64)
    with pytest.raises(ValueError):
        pack_slab(K, np.zeros((32, 64), np.float32), "f32", 4, 2, 0, 0, v_group=48)


# ----------------------------------------------------------------- key group length
# Keys are quantized per channel over k_group = 32 (default), 64 or 128 consecutive
# quantized tokens; codes keep their 32-token groups.  Pinned the same way: a closed
# form with one key group for the whole cache, an exact reduction to the pinned
# 32-token grouping, and the half-step bound.

def _k_rows(rng, T, Dk):
    return (rng.standard_normal((T, Dk)) * 2 + 1).astype(np.float32)


@pytest.mark.parametrize("kb", [2, 3, 4, 8])
def test_whole_cache_key_group_closed_form(kb):
    rng = np.random.default_rng(41)
    T, Dk, Dv = 128, 64, 32
    K = _k_rows(rng, T, Dk)
    V = _v_rows(rng, T, Dv)
    p = pack_slab(K, V, "f32", kb, 2, 0, 0, k_group=128)
    assert p["k_scale"].shape == (1, Dk) and p["k_codes"].shape == (T, Dk * kb // 32)
    levels = np.float32(2 ** kb - 1)
    want_s = ((K.max(axis=0) - K.min(axis=0)) / levels).astype(np.float16)
    want_z = K.min(axis=0).astype(np.float16)
    assert np.array_equal(p["k_scale"][0], want_s.view(np.uint16))
    assert np.array_equal(p["k_zero"][0], want_z.view(np.uint16))


@pytest.mark.parametrize("kb", [2, 4])
def test_64_key_group_reduces_to_32_when_halves_share_range(kb):
    rng = np.random.default_rng(42)
    T, Dk, Dv = 192, 64, 32
    K = _k_rows(rng, T, Dk)
    V = _v_rows(rng, T, Dv)
    lo, hi = K.min(axis=0) - 1.0, K.max(axis=0) + 1.0
    for g0 in range(0, T, 64):            # both 32-token halves of every 64-group reach lo and hi
        for h0 in (g0, g0 + 32):
            K[h0 + 5] = lo
            K[h0 + 20] = hi
    p32 = pack_slab(K, V, "f32", kb, 2, 0, 0, k_group=32)
    p64 = pack_slab(K, V, "f32", kb, 2, 0, 0, k_group=64)
    assert np.array_equal(p32["k_codes"], p64["k_codes"])
    for key in ("k_scale", "k_zero"):
        assert np.array_equal(p32[key][0::2], p64[key]) and np.array_equal(p32[key][1::2], p64[key])
    for key in ("v_codes", "v_scale", "v_zero"):
        assert np.array_equal(p32[key], p64[key])


@pytest.mark.parametrize("kg", [32, 64, 128])
def test_key_dequant_within_half_step(kg):
    rng = np.random.default_rng(43)
    T, Dk, Dv, kb = 256, 64, 32, 4
    K = _k_rows(rng, T, Dk)
    V = _v_rows(rng, T, Dv)
    p = pack_slab(K, V, "f32", kb, 2, 0, 0, k_group=kg)
    Khat, _ = dequant_slab(p, kb, 2)
    s = np.repeat(p["k_scale"].view(np.float16).astype(np.float64), kg, axis=0)
    z = np.repeat(p["k_zero"].view(np.float16).astype(np.float64), kg, axis=0)
    mn = np.repeat(K.reshape(T // kg, kg, Dk).min(axis=1).astype(np.float64), kg, axis=0)
    assert np.all(np.abs(Khat - K.astype(np.float64)) <= 0.5 * s + np.abs(z - mn) + 1e-6)


def test_bad_key_group():
    with pytest.raises(ValueError):
        pack_slab(np.zeros((96, 32), np.float32), np.zeros((96, 32), np.float32), "f32", 4, 2, 0, 0, k_group=64)
    with pytest.raises(ValueError):
        pack_slab(np.zeros((64, 32), np.float32), np.zeros((64, 32), np.float32), "f32", 4, 2, 0, 0, k_group=48)


# ------------------------------------------------------------------- 1-bit codes
# With one bit, the quantizer contract reduces to a threshold: code = rint(t) clamped
# to [0, 1] with t = (x - z) / s, i.e. 1 exactly when t > 0.5 (rint sends 0.5 to the
# even 0).  Key words are plain little-endian bit strings along the channels, which
# numpy's packbits writes out independently.

@pytest.mark.parametrize("seed", [51, 52])
def test_one_bit_codes_are_a_threshold(seed):
    from oracle import quantize_groups
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((40, 32)) * 3).astype(np.float32)
    x[0, :] = np.linspace(-1, 1, 32, dtype=np.float32)            # includes exact midpoints
    codes, s16, z16 = quantize_groups(x, 1)
    s = s16.astype(np.float32)[:, None]
    z = z16.astype(np.float32)[:, None]
    t = (x - z) / s
    assert np.array_equal(codes, (t > np.float32(0.5)).astype(np.uint8))


def test_one_bit_key_words_match_packbits():
    from oracle import pack_codes
    rng = np.random.default_rng(53)
    codes = rng.integers(0, 2, size=(7, 96), dtype=np.uint8)
    words = pack_codes(codes, 1)
    want = np.packbits(codes, axis=1, bitorder="little").view("<u4")
    assert np.array_equal(words, want)


@pytest.mark.parametrize("Dv", [32, 64, 128])
def test_one_bit_value_layout(Dv):
    from oracle import pack_value_codes, unpack_value_codes, value_bit_position
    tau, c = np.meshgrid(np.arange(32), np.arange(Dv), indexing="ij")
    pos = value_bit_position(tau, c, Dv, 1)
    assert np.array_equal(np.sort(pos.ravel()), np.arange(32 * Dv))  # one bit per code, no gaps
    # hand-derived at Dv = 128 (one 16-bit field per (octet, column, pair): 8 tiles of the first
    # token of the pair, then 8 of the second): token 13 = octet 1, j = 5; channel 37 = tile 2, column 5
    if Dv == 128:
        assert value_bit_position(13, 37, 128, 1) == ((16 * 1 + 5) * 4 + 1) * 16 + 8 + 2
        assert value_bit_position(0, 0, 128, 1) == 0 and value_bit_position(4, 0, 128, 1) == 8
    rng = np.random.default_rng(54)
    codes = rng.integers(0, 2, size=(3, 32, Dv), dtype=np.uint8)
    assert np.array_equal(unpack_value_codes(pack_value_codes(codes, 1), 1), codes)


def test_one_bit_pack_slab_round_trip():
    rng = np.random.default_rng(55)
    T, Dk, Dv = 96, 64, 128
    K = rng.standard_normal((T, Dk)).astype(np.float32)
    V = rng.standard_normal((T, Dv)).astype(np.float32)
    p = pack_slab(K, V, "f32", 1, 1, 32, 0)
    assert p["k_codes"].shape == (64, 2) and p["v_codes"].shape == (2, 128)
    Khat, Vhat = dequant_slab(p, 1, 1)
    ks = np.repeat(p["k_scale"].view(np.float16).astype(np.float64), 32, axis=0)
    assert np.all(np.abs(Khat[:64] - K[:64]) <= 0.5 * ks + 1e-2)


# ------------------------------------------------------------------- 3-bit codes
# 32 is not a multiple of 3, so 3-bit codes are plain little-endian bit streams and a
# code may straddle two words: key row bit 3c holds channel c; a value group's stream
# holds (token tau, channel c) at bit 3 (tau Dv + c).  Pinned against streams built
# as one Python integer per row (sum of code << position), cut into 32-bit words.

def _words_of_int(v, n_words):
    return np.array([(v >> (32 * k)) & 0xFFFFFFFF for k in range(n_words)], dtype=np.uint32)


@pytest.mark.parametrize("n", [32, 96, 128, 256])
def test_three_bit_key_rows_are_bit_streams(n):
    from oracle import pack_codes, unpack_codes
    rng = np.random.default_rng(60 + n)
    codes = rng.integers(0, 8, size=(5, n), dtype=np.uint8)
    codes[0, 10] = 7                                  # bits 30..32: straddles words 0 and 1
    words = pack_codes(codes, 3)
    assert words.shape == (5, 3 * n // 32)
    for r in range(5):
        v = sum(int(c) << (3 * k) for k, c in enumerate(codes[r]))
        assert np.array_equal(words[r], _words_of_int(v, 3 * n // 32))
    assert (words[0, 0] >> 30) & 3 == 3 and words[0, 1] & 1 == 1
    assert np.array_equal(unpack_codes(words, 3), codes)


@pytest.mark.parametrize("Dv", [32, 96, 128])
def test_three_bit_value_stream(Dv):
    from oracle import pack_value_codes, unpack_value_codes, value_bit_position
    tau, c = np.meshgrid(np.arange(32), np.arange(Dv), indexing="ij")
    pos = value_bit_position(tau, c, Dv, 3)
    assert np.array_equal(np.sort(pos.ravel()), np.arange(0, 96 * Dv, 3))   # token-major, no gaps
    assert value_bit_position(1, 2, Dv, 3) == 3 * (Dv + 2)
    rng = np.random.default_rng(70 + Dv)
    codes = rng.integers(0, 8, size=(2, 32, Dv), dtype=np.uint8)
    words = pack_value_codes(codes, 3)
    assert words.shape == (2, 3 * Dv)
    for g in range(2):
        v = sum(int(codes[g, t, ch]) << (3 * (t * Dv + ch)) for t in range(32) for ch in range(Dv))
        assert np.array_equal(words[g], _words_of_int(v, 3 * Dv))
    assert np.array_equal(unpack_value_codes(words, 3), codes)


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (96, 64)])
def test_three_bit_pack_slab_within_half_step(Dk, Dv):
    rng = np.random.default_rng(80)
    T = 96
    K = (rng.standard_normal((T, Dk)) * 2 + 1).astype(np.float32)
    V = rng.standard_normal((T, Dv)).astype(np.float32)
    p = pack_slab(K, V, "f32", 3, 3, 32, 0)
    assert p["k_codes"].shape == (64, 3 * Dk // 32) and p["v_codes"].shape == (2, 3 * Dv)
    Khat, Vhat = dequant_slab(p, 3, 3)
    ks = np.repeat(p["k_scale"].view(np.float16).astype(np.float64), 32, axis=0)
    kz = np.repeat(p["k_zero"].view(np.float16).astype(np.float64), 32, axis=0)
    kmin = np.repeat(K[:64].reshape(2, 32, Dk).min(axis=1).astype(np.float64), 32, axis=0)
    assert np.all(np.abs(Khat[:64] - K[:64]) <= 0.5 * ks + np.abs(kz - kmin) + 1e-6)
    vs = p["v_scale"].view(np.float16).astype(np.float64).transpose(0, 2, 1).reshape(64, Dv // 32)
    vz = p["v_zero"].view(np.float16).astype(np.float64).transpose(0, 2, 1).reshape(64, Dv // 32)
    vmin = V[:64].reshape(64, Dv // 32, 32).min(axis=2).astype(np.float64)
    err = np.abs(Vhat[:64] - V[:64]).reshape(64, Dv // 32, 32)
    assert np.all(err <= (0.5 * vs + np.abs(vz - vmin))[:, :, None] + 1e-6)
    assert unpack_codes(p["k_codes"], 3).max() == 7
