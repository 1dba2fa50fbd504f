"""HeadQ side code over the packed cache (CPU oracle; TEST INFRASTRUCTURE ONLY: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the HIP library never calls it and shares nothing with it).

Source: "HeadQ" technical summary, section 3 (methodology).  Write path: the low-bit
quantizer gives the base key k_hat_j; the residual e_j = k_j - k_hat_j is projected
on a rank-r basis U_h of the head and stored as a low-bit side code
z_j = Q_q(U_h^T e_j).  Read path: the current query turns the side code into an
additive logit correction, s_j = q.k_hat_j / sqrt(d) + q.(U_h z_hat_j) / sqrt(d).

Readings where the page leaves a step open (parity of the mechanics only):

* U_h is an input, fp32 [Dk, r] per KV head.  The page learns it by PCA on
  calibration queries; no calibration data exists here, and any basis exercises
  the same arithmetic.
* Q_q is the library's asymmetric min/max quantizer (``quantize_groups``) applied
  to the r coefficients of one token as one group, with side_bits bits and fp16
  scale and zero; z_hat = code * s + z.
* U_h^T e_j is accumulated in float64 over channels in ascending order (no fused
  multiply-add) and rounded once to float32, the precision the quantizer works in.
* Only quantized tokens carry a side code: fp16-retained tokens have no residual
  worth coding.
"""

import numpy as np

from .kvq_oracle import dequant_slab, quantize_groups, split_positions, upcast, attention


def project_residual(K_rows, Khat_rows, U):
    """y = U^T (k - k_hat) per row, float64, channels summed in ascending order.
    K_rows float32 [n, Dk], Khat_rows float64 [n, Dk], U float32 [Dk, r] -> [n, r]."""
    e = np.asarray(K_rows, dtype=np.float64) - np.asarray(Khat_rows, dtype=np.float64)
    U64 = np.asarray(U, dtype=np.float32).astype(np.float64)
    y = np.zeros((e.shape[0], U64.shape[1]), dtype=np.float64)
    for c in range(e.shape[1]):
        y = y + e[:, c:c + 1] * U64[c][None, :]
    return y


def side_code(K_rows, Khat_rows, U, side_bits: int):
    """(codes uint8 [n, r], scale fp16 [n], zero fp16 [n]) of the residual projections."""
    y = project_residual(K_rows, Khat_rows, U).astype(np.float32)
    return quantize_groups(y, side_bits)


def headq_side_slab(K, dtype: str, p, U, k_bits: int, v_bits: int, n_recent: int, log_window: int,
                    side_bits: int):
    """Side code of every quantized token of one packed slab (compacted order).
    K [T, Dk] in storage dtype; p = pack_slab of the same slab."""
    _, u = split_positions(K.shape[0], n_recent, log_window)
    Khat, _ = dequant_slab(p, k_bits, v_bits)
    codes, s16, z16 = side_code(upcast(K, dtype)[u], Khat[:len(u)], U, side_bits)
    return {"side_codes": codes.astype(np.uint8), "side_scale": s16.view(np.uint16),
            "side_zero": z16.view(np.uint16)}


def corrected_keys(p, side, U, k_bits: int, v_bits: int):
    """Keys as the read path sees them: k_hat_j + U z_hat_j for quantized tokens, the
    fp16 rows unchanged; returned with the dequantized values."""
    Khat, Vhat = dequant_slab(p, k_bits, v_bits)
    zc = side["side_codes"].astype(np.float64)
    zs = side["side_scale"].view(np.float16).astype(np.float64)[:, None]
    zz = side["side_zero"].view(np.float16).astype(np.float64)[:, None]
    zhat = zc * zs + zz                                              # [Tq, r]
    K = Khat.copy()
    K[:zhat.shape[0]] += zhat @ np.asarray(U, dtype=np.float32).astype(np.float64).T
    return K, Vhat


def decode_slab_headq(q_group, p, side, U, q_dtype: str, k_bits: int, v_bits: int, scale):
    """Decode attention of the G query heads of one KV head with the logit correction:
    q.(k_hat_j + U z_hat_j) = q.k_hat_j + (U^T q).z_hat_j, scaled."""
    K, V = corrected_keys(p, side, U, k_bits, v_bits)
    return attention(upcast(q_group, q_dtype), K, V, scale)
