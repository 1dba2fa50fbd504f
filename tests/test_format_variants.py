"""Pins of the value-group width (CPU only).

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

from oracle import dequant_slab, pack_slab, unpack_value_codes


def _v_rows(rng, T, Dv):
    return (rng.standard_normal((T, Dv)) * 0.5).astype(np.float32)


@pytest.mark.parametrize("vb", [2, 4, 8])
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
