"""Pins of the HeadQ side-code oracle (CPU only).

"HeadQ" (section 3): residual e_j = k_j - k_hat_j, side code z_j = Q_q(U^T e_j), logit
correction q.U z_hat_j / sqrt(d).  Pinned against:

* a hand-computed example (Dk = 2, rank 1);
* the degenerate case of keys already on the quantization grid: zero residual, zero
  side code, decode equal to the plain packed decode;
* the identity basis (r = Dk): corrected keys lie within half a side step (plus the
  fp16 rounding of the zero) of the original keys;
* queries inside span(U) (orthonormal U from a seeded QR): the correction removes most
  of the score error, and the wrong-sign correction makes it worse than none, the
  page's directionality control;
* the sequential float64 projection against numpy's matrix product.
"""

import numpy as np
import pytest

import oracle as O


def test_hand_example_rank_one():
    K = np.array([[1.0, 2.0]], np.float32)
    Khat = np.array([[0.5, 1.5]], np.float64)                # e = (0.5, 0.5)
    U = np.array([[0.6], [0.8]], np.float32)                  # y = 0.5 * 0.6 + 0.5 * 0.8 = 0.7
    codes, s16, z16 = O.side_code(K, Khat, U, 8)
    assert codes.shape == (1, 1) and codes[0, 0] == 0           # one coefficient: max == min, s = 0
    assert s16[0] == 0 and z16[0] == np.float16(np.float32(0.5) * np.float32(0.6) + np.float32(0.5) * np.float32(0.8))
    assert float(z16[0]) == 0.7001953125


def _slab(rng, T, Dk, Dv):
    K = (rng.standard_normal((T, Dk)) * 1.5).astype(np.float32)
    V = rng.standard_normal((T, Dv)).astype(np.float32)
    return K, V


def test_keys_on_the_grid_give_a_zero_side_code():
    rng = np.random.default_rng(90)
    T, Dk, Dv = 96, 32, 32
    # every channel of every 32-token group takes only the values 0 and 3 (2-bit grid, s = 1, z = 0)
    K = (rng.integers(0, 2, size=(T, Dk)) * 3).astype(np.float32)
    K[0::32] = 0.0
    K[1::32] = 3.0
    V = rng.standard_normal((T, Dv)).astype(np.float32)
    p = O.pack_slab(K, V, "f32", 2, 2, 0, 0)
    U = np.linalg.qr(rng.standard_normal((Dk, 4)))[0].astype(np.float32)
    side = O.headq_side_slab(K, "f32", p, U, 2, 2, 0, 0, 8)
    assert not side["side_codes"].any() and not side["side_scale"].any() and not side["side_zero"].any()
    q = rng.standard_normal((2, Dk)).astype(np.float32)
    got = O.decode_slab_headq(q, p, side, U, "f32", 2, 2, 0.25)
    assert np.array_equal(got, O.decode_slab(q, p, "f32", 2, 2, 0.25))


@pytest.mark.parametrize("bits", [4, 8])
def test_identity_basis_bounds_the_key_error(bits):
    rng = np.random.default_rng(91)
    T, Dk, Dv = 128, 32, 32
    K, V = _slab(rng, T, Dk, Dv)
    p = O.pack_slab(K, V, "f32", 2, 2, 32, 0)
    U = np.eye(Dk, dtype=np.float32)
    side = O.headq_side_slab(K, "f32", p, U, 2, 2, 32, 0, bits)
    Kc, _ = O.corrected_keys(p, side, U, 2, 2)
    Khat, _ = O.dequant_slab(p, 2, 2)
    e = K[:96].astype(np.float64) - Khat[:96]
    s = side["side_scale"].view(np.float16).astype(np.float64)[:, None]
    z = side["side_zero"].view(np.float16).astype(np.float64)[:, None]
    bound = 0.5 * s + np.abs(z - e.astype(np.float32).min(axis=1, keepdims=True)) + 1e-6
    assert np.all(np.abs(Kc[:96] - K[:96]) <= bound)
    assert np.abs(Kc[:96] - K[:96]).max() < 0.25 * np.abs(e).max()


def test_in_span_queries_and_the_sign_of_the_correction():
    rng = np.random.default_rng(92)
    T, Dk, Dv, r = 320, 64, 64, 4
    K, V = _slab(rng, T, Dk, Dv)
    p = O.pack_slab(K, V, "f32", 2, 2, 0, 0)
    U = np.linalg.qr(rng.standard_normal((Dk, r)))[0].astype(np.float32)
    side = O.headq_side_slab(K, "f32", p, U, 2, 2, 0, 0, 8)
    q = (U.astype(np.float64) @ rng.standard_normal((r, 3))).T      # queries inside span(U)
    Khat, _ = O.dequant_slab(p, 2, 2)
    Kc, _ = O.corrected_keys(p, side, U, 2, 2)
    exact = q @ K.astype(np.float64).T
    err_base = np.abs(q @ Khat.T - exact).max()
    err_corr = np.abs(q @ Kc.T - exact).max()
    err_wrong = np.abs(q @ (2 * Khat - Kc).T - exact).max()          # the correction subtracted
    assert err_corr < 0.05 * err_base
    assert err_wrong > err_base


def test_sequential_projection_matches_matmul():
    rng = np.random.default_rng(93)
    K = rng.standard_normal((50, 128)).astype(np.float32)
    Khat = rng.standard_normal((50, 128))
    U = rng.standard_normal((128, 8)).astype(np.float32)
    y = O.project_residual(K, Khat, U)
    want = (K.astype(np.float64) - Khat) @ U.astype(np.float64)
    assert np.allclose(y, want, rtol=0, atol=1e-11)
