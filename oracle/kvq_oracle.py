"""CPU oracle: group-wise asymmetric low-bit KV cache + single-token decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library never
calls it, and it shares no code, constant or table with the HIP library.

Plain NumPy, written for a reader to check against the pages by eye:

* quantize side in float32 with round-half-to-even, exactly as spelled out in
  ``quantize_groups``;
* dequantization and attention in float64.

Sources (the pages are secondary machine-written summaries; where they leave a step
open the plainest reading is taken and listed in the design notes):

* "Quantize What Counts: More for Keys, Less for Values" (technical summary,
  methodology / results): keys and values take separate bit widths (K4V2), group
  size 32 for keys.
* "LogQuant: Log-Distributed 2-Bit Quantization of KV Cache" (technical summary,
  section 2 "log-based filtering strategy", section 4 "position-independent
  optimisation", section 5 "implementation"): newest tokens kept in full
  precision, log-spaced full-precision tokens further back, per-channel key
  quantization, attention over an arbitrary concatenation of full-precision and
  quantized tokens (A.V = A_P.V_P).
* "HeadQ" (section 2.1): score s_j = q^T k_j / sqrt(d); a constant vector added to
  every key shifts every score by the same amount (softmax-null direction).
* "Thin Keys, Full Values" (section 2): softmax(Q K^T / sqrt(d_select)) V with
  d_select (key width) different from the value width.
* "Quantize What Counts" (technical summary, contributions "orthogonality and
  integration" and results "rotation integration"): an optional rotation of the
  keys only before they are quantized, to spread outlier channels; the pages name
  rotation-based outlier redistribution without fixing the transform, read here as
  the orthonormal Walsh-Hadamard transform (``hadamard_rotate``), applied to every
  key row (quantized or kept in fp16) and, at decode, to the query, so that
  scores are unchanged in exact arithmetic.

Canonical packed layout for one (b, kv-head) slab (the same index formulas appear in
``include/kvq.h``; the oracle writes them out here independently):

* retained (fp16) positions r = sorted retained set, compacted positions
  u = sorted(the rest); Tq = len(u), groups of 32 consecutive compacted tokens;
* k_codes  u32 [Tq, Dk*kb/32]: word w of row t holds channel w*(32/kb)+k at bits
  [k*kb, k*kb+kb), little-endian (keys stored token by token);
* k_scale, k_zero fp16 [Tq/gK, Dk]  (one pair per key group of gK = 32 (default),
  64 or 128 tokens and channel; codes still come in 32-token groups);
* v_codes  u32 [Tq/32, Dv*vb]: each 32-token group's value codes form one
  little-endian bit stream (bit i of the stream is bit i%32 of word i/32); the
  code of token 8o+j of the group (octet o, j < 8) and channel c = 16t+n (tile t,
  column n < 16) sits at bit
      ((16o + n)*4 + j%4)*F + chunk*32 + (j//4)*r*vb + (t%TPW)*vb,
  with TPW = 16/vb tiles per chunk, chunk = t//TPW, r = min(TPW, Dv/16 - chunk*TPW)
  tiles in that chunk and F = Dv*vb/8 bits per (o, n, j%4) field: one field pairs
  tokens j and j+4 of an octet, the first of them in the low half of every chunk
  (library format choice, see ``value_bit_position``);
* 3-bit codes (32 is not a multiple of 3) are plain little-endian bit streams
  instead, so a code may straddle two words: key row t holds channel c at stream
  bits [3c, 3c+3), and a group's value stream holds token tau, channel c at bits
  [3(tau*Dv + c), 3(tau*Dv + c) + 3);
* v_scale, v_zero fp16 [Tq/32, Dv/gV, 32]  (one pair per token and gV-channel
  group, gV = 32 by default, the 32 tokens of a group contiguous);
* k_fp16 [R, Dk], v_fp16 [R, Dv] fp16 rows of the retained positions, ascending.
"""

import numpy as np

GROUP = 32  # tokens per key group and channels per value group


# ----------------------------------------------------------------------------- inputs

def upcast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage dtype -> float32, exactly.  bf16 arrives as uint16 bit patterns: a bf16
    number is the upper half of the float32 with the same bits."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float32)
    raise ValueError(dtype)


def default_scale(Dk: int) -> np.float32:
    """Softmax scale 1/sqrt(d) of the score s = q^T k / sqrt(d) (HeadQ 2.1; Thin Keys 2,
    with d the key width), as one float32 value."""
    return np.float32(1.0) / np.sqrt(np.float32(Dk))


# -------------------------------------------------------------------------- rotation

def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform (Sylvester order) along the last axis,
    in float32 with one fixed order of operations: butterflies for h = 1, 2, 4, ...,
    n/2 (entries j and j + h of every 2h-block become a + b and a - b), then one
    multiply by fp32(2^(-m/2)) for n = 2^m, i.e. fp32(sqrt(1/2)) * 2^(-(m-1)/2) for
    odd m.  Any implementation that takes the same steps gets the same bits."""
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    m = n.bit_length() - 1
    if n != 1 << m:
        raise ValueError("rotation needs a power-of-two width, got %d" % n)
    lead = y.shape[:-1]
    h = 1
    while h < n:
        v = y.reshape(lead + (n // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        y = v.reshape(lead + (n,))
        h *= 2
    c = np.float32(2.0 ** -(m // 2))
    if m % 2:
        c = np.float32(np.float32(np.sqrt(0.5)) * c)
    return (y * c).astype(np.float32)


# ------------------------------------------------------------------------- retention

def retained_mask(T: int, n_recent: int, log_window: int) -> np.ndarray:
    """Which of the T cached positions stay in fp16 (LogQuant section 2).

    * the newest ``n_recent`` positions;
    * with W = log_window > 0, for j = 1, 2, ...: inside the span
      [T - W*2^j, T - W*2^(j-1)) (clipped at 0), every position that is a multiple
      of 2^j.  Going one span back doubles both the span and the stride: every 2nd
      token in [T-2W, T-W), every 4th in [T-4W, T-2W), and so on.
    """
    keep = np.zeros(T, dtype=bool)
    keep[max(0, T - n_recent):] = True
    if log_window > 0:
        j = 1
        while T - log_window * 2 ** (j - 1) > 0:
            hi = T - log_window * 2 ** (j - 1)
            lo = max(0, T - log_window * 2 ** j)
            pos = np.arange(lo, hi)
            keep[pos[pos % 2 ** j == 0]] = True
            j += 1
    return keep


def split_positions(T: int, n_recent: int, log_window: int):
    """(retained positions r, quantized positions u), both ascending (LogQuant section 4:
    the two sets are stored apart; the order inside attention does not matter)."""
    keep = retained_mask(T, n_recent, log_window)
    return np.nonzero(keep)[0], np.nonzero(~keep)[0]


# ---------------------------------------------------------------------- quantization

def quantize_groups(x: np.ndarray, bits: int):
    """Asymmetric min/max quantization of each group along the last axis.

    x float32 [..., n].  For each group (all float32, IEEE rounding):
        mn, mx = min x, max x
        s = fp16(fp32(mx - mn) / fp32(2^bits - 1))     (round to nearest even)
        z = fp16(mn)
        code = clamp(rint((x - z_f32) / s_f32), 0, 2^bits - 1), rint ties to even;
        code = 0 everywhere when s == 0.
    A stored zero of either sign is written as +0.
    Returns codes uint8 [..., n], s and z as float16 [...].
    """
    x = np.asarray(x, dtype=np.float32)
    levels = np.float32(2 ** bits - 1)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    s16 = ((mx - mn) / levels).astype(np.float16)
    z16 = mn.astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(0.0), s16)
    z16 = np.where(z16 == 0, np.float16(0.0), z16)
    s = s16.astype(np.float32)[..., None]
    z = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - z) / s
    codes = np.where(s == 0, np.float32(0), np.clip(np.rint(t), np.float32(0), levels))
    return codes.astype(np.uint8), s16, z16


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., n] -> uint32 [..., n*bits/32]; code k of each word at bits [k*bits, k*bits+bits).
    3-bit codes: code c at bits [3c, 3c+3) of the row's little-endian bit stream."""
    if bits == 3:
        return _stream_pack(codes, 3)
    per = 32 // bits
    c = np.asarray(codes, dtype=np.uint32)
    c = c.reshape(c.shape[:-1] + (c.shape[-1] // per, per))
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    return np.bitwise_or.reduce(c << shifts, axis=-1).astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_codes: uint32 [..., w] -> uint8 [..., w*32/bits]."""
    if bits == 3:
        return _stream_unpack(words, 3)
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint32)[..., None]
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    c = (w >> shifts) & np.uint32(2 ** bits - 1)
    return c.reshape(c.shape[:-2] + (c.shape[-2] * per,)).astype(np.uint8)


def _stream_pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., n] -> uint32 [..., n*bits/32]: code k at bits [k*bits, (k+1)*bits)
    of a little-endian bit stream (bit i of the stream = bit i%32 of word i/32)."""
    c = np.asarray(codes, dtype=np.uint32)
    n = c.shape[-1]
    if (n * bits) % 32:
        raise ValueError("a %d-bit stream of %d codes is not a whole number of words" % (bits, n))
    planes = (c[..., :, None] >> np.arange(bits, dtype=np.uint32)) & np.uint32(1)   # [..., n, bits]
    stream = planes.reshape(c.shape[:-1] + (n * bits // 32, 32))                      # bit i at [i/32, i%32]
    return (stream << np.arange(32, dtype=np.uint32)).sum(axis=-1, dtype=np.uint64).astype(np.uint32)


def _stream_unpack(words: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of _stream_pack: uint32 [..., w] -> uint8 [..., w*32/bits]."""
    w = np.asarray(words, dtype=np.uint32)
    stream = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)     # [..., w, 32]
    planes = stream.reshape(w.shape[:-1] + (w.shape[-1] * 32 // bits, bits))
    return (planes << np.arange(bits, dtype=np.uint32)).sum(axis=-1).astype(np.uint8)


def value_bit_position(tau, c, Dv: int, bits: int):
    """Bit offset, inside its group's value bit stream, of the code of token tau
    (0..31 within the group) and channel c (library format choice; documented in the
    module header).  Works elementwise on integer arrays."""
    tau = np.asarray(tau, dtype=np.int64)
    c = np.asarray(c, dtype=np.int64)
    if bits == 3:                              # plain token-major stream
        return 3 * (tau * Dv + c)
    n_tiles = Dv // 16
    per_chunk = 16 // bits                     # tiles whose codes share one chunk
    field = Dv * bits // 8                     # bits per (octet, column, token pair)
    octet, j = tau // 8, tau % 8
    pair, upper = j % 4, j // 4
    col, tile = c % 16, c // 16
    chunk, slot = tile // per_chunk, tile % per_chunk
    in_chunk = np.minimum(per_chunk, n_tiles - chunk * per_chunk)
    return (((octet * 16 + col) * 4 + pair) * field + chunk * 2 * per_chunk * bits
            + upper * in_chunk * bits + slot * bits)


def pack_value_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., 32, Dv] (token, channel of one group) -> uint32 [..., Dv*bits]."""
    c = np.asarray(codes, dtype=np.uint64)
    Dv = c.shape[-1]
    if c.shape[-2] != GROUP or Dv % GROUP:
        raise ValueError("value codes must be [..., 32, Dv] with Dv a multiple of 32")
    tau, ch = np.meshgrid(np.arange(GROUP), np.arange(Dv), indexing="ij")
    pos = value_bit_position(tau, ch, Dv, bits).reshape(-1)
    assert np.unique(pos).size == pos.size and pos.max() < GROUP * Dv * bits
    lead = c.shape[:-2]
    flat = c.reshape((-1, GROUP * Dv))
    words = np.zeros((flat.shape[0], Dv * bits), dtype=np.uint64)
    for row in range(flat.shape[0]):
        # disjoint fields: adding each code at its position is the same as OR-ing it in
        np.add.at(words[row], pos // 32, flat[row] << (pos % 32).astype(np.uint64))
    # a 3-bit code may straddle two words: its bits past 31 belong to the next word
    carry = words >> np.uint64(32)
    words &= np.uint64(0xFFFFFFFF)
    words[:, 1:] += carry[:, :-1]
    assert not carry[:, -1].any()
    return words.astype(np.uint32).reshape(lead + (Dv * bits,))


def unpack_value_codes(words: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_value_codes: uint32 [..., Dv*bits] -> codes uint8 [..., 32, Dv]."""
    w = np.asarray(words, dtype=np.uint64)
    Dv = w.shape[-1] // bits
    tau, ch = np.meshgrid(np.arange(GROUP), np.arange(Dv), indexing="ij")
    pos = value_bit_position(tau, ch, Dv, bits)
    # each word joined with the next one (zero past the end): a 3-bit code may straddle two
    nxt = np.concatenate([w[..., 1:], np.zeros(w.shape[:-1] + (1,), np.uint64)], axis=-1)
    w = w | (nxt << np.uint64(32))
    codes = (w[..., pos // 32] >> (pos % 32).astype(np.uint64)) & np.uint64(2 ** bits - 1)
    return codes.astype(np.uint8)


def pack_slab(K, V, dtype: str, k_bits: int, v_bits: int, n_recent: int, log_window: int,
              key_rotation: bool = False, v_group: int = GROUP, k_group: int = GROUP):
    """Quantize and pack one (b, kv-head) slab.  K [T, Dk], V [T, Dv] in storage dtype.

    Keys per channel over groups of k_group consecutive quantized tokens (LogQuant
    section 5, "per-channel" keys; group 32 by default from "Quantize What Counts",
    results, which also sweeps the group size); values per token over groups of
    v_group channels (32 by default); retained positions copied to fp16.
    With key_rotation every key row is first rotated (``hadamard_rotate``).
    """
    K32 = upcast(K, dtype)
    if key_rotation:
        K32 = hadamard_rotate(K32)
    V32 = upcast(V, dtype)
    T, Dk = K32.shape
    Dv = V32.shape[1]
    r, u = split_positions(T, n_recent, log_window)
    Tq = len(u)
    if Dk % GROUP or Dv % GROUP:
        raise ValueError("head widths must be multiples of %d" % GROUP)
    if v_group not in (32, 64, 128) or Dv % v_group:
        raise ValueError("value group %d must be 32, 64 or 128 and divide Dv = %d" % (v_group, Dv))
    if k_group not in (32, 64, 128):
        raise ValueError("key group %d must be 32, 64 or 128" % k_group)
    if Tq % k_group:
        raise ValueError("quantized token count %d is not a multiple of %d" % (Tq, k_group))
    nG = Tq // GROUP

    # keys: key group g = compacted tokens k_group g .. k_group g + k_group - 1, one
    # (s, z) per channel
    Kg = K32[u].reshape(Tq // k_group, k_group, Dk).transpose(0, 2, 1)   # [Tq/gK, Dk, gK]
    kc, ks, kz = quantize_groups(Kg, k_bits)                              # [Tq/gK, Dk, gK], [Tq/gK, Dk]
    kc = kc.transpose(0, 2, 1).reshape(Tq, Dk)
    # values: one (s, z) per token and v_group-channel group
    Vg = V32[u].reshape(Tq, Dv // v_group, v_group)
    vc, vs, vz = quantize_groups(Vg, v_bits)                          # [Tq, Dv/gV, gV], [Tq, Dv/gV]
    vc = vc.reshape(nG, GROUP, Dv)                                     # [nG, 32 tokens, Dv]
    vs = vs.reshape(nG, GROUP, Dv // v_group).transpose(0, 2, 1)     # [nG, Dv/gV, 32]
    vz = vz.reshape(nG, GROUP, Dv // v_group).transpose(0, 2, 1)

    return {
        "k_codes": pack_codes(kc, k_bits),
        "k_scale": ks.view(np.uint16),
        "k_zero": kz.view(np.uint16),
        "v_codes": pack_value_codes(vc, v_bits),
        "v_scale": np.ascontiguousarray(vs).view(np.uint16),
        "v_zero": np.ascontiguousarray(vz).view(np.uint16),
        "k_fp16": K32[r].astype(np.float16).view(np.uint16),
        "v_fp16": V32[r].astype(np.float16).view(np.uint16),
    }


CACHE_KEYS = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_fp16", "v_fp16")


def pack_all(K, V, w):
    """pack_slab over every (b, h); returns arrays with leading [B, Hkv] axes."""
    out = {key: [] for key in CACHE_KEYS}
    for b in range(K.shape[0]):
        rows = {key: [] for key in CACHE_KEYS}
        for h in range(K.shape[1]):
            p = pack_slab(K[b, h], V[b, h], w.dtype, w.k_bits, w.v_bits, w.n_recent, w.log_window,
                          getattr(w, "key_rotation", False), getattr(w, "v_group", GROUP),
                          getattr(w, "k_group", GROUP))
            for key in CACHE_KEYS:
                rows[key].append(p[key])
        for key in CACHE_KEYS:
            out[key].append(np.stack(rows[key]))
    return {key: np.stack(v) for key, v in out.items()}


# ---------------------------------------------------------------------- dequant + attn

def dequant_slab(p, k_bits: int, v_bits: int):
    """float64 keys and values of one packed slab: quantized tokens (compacted order)
    followed by the retained fp16 tokens.  x_hat = code * s + z (exact in float64).
    The key group length is read off the key scale array (Tq / its first axis), the
    value group width off the value scale array (Dv / its second axis)."""
    kc = unpack_codes(p["k_codes"], k_bits).astype(np.float64)      # [Tq, Dk]
    Tq, Dk = kc.shape
    ks = p["k_scale"].view(np.float16).astype(np.float64)            # [Tq/gK, Dk]
    kz = p["k_zero"].view(np.float16).astype(np.float64)
    g = np.arange(Tq) // (Tq // ks.shape[0]) if ks.shape[0] else np.zeros(0, np.int64)
    Khat_q = kc * ks[g] + kz[g]
    vc = unpack_value_codes(p["v_codes"], v_bits)                    # [nG, 32, Dv]
    nG, _, Dv = vc.shape
    vc = vc.reshape(Tq, Dv).astype(np.float64)                       # token 32g + t
    ngv = p["v_scale"].shape[1]                                      # Dv / v_group
    vs = p["v_scale"].view(np.float16).astype(np.float64).transpose(0, 2, 1).reshape(Tq, ngv)
    vz = p["v_zero"].view(np.float16).astype(np.float64).transpose(0, 2, 1).reshape(Tq, ngv)
    Vhat_q = vc * np.repeat(vs, Dv // ngv, axis=1) + np.repeat(vz, Dv // ngv, axis=1)
    Kr = p["k_fp16"].view(np.float16).astype(np.float64)              # [R, Dk]
    Vr = p["v_fp16"].view(np.float16).astype(np.float64)              # [R, Dv]
    return np.concatenate([Khat_q, Kr]), np.concatenate([Vhat_q, Vr])


def attention(q, K, V, scale) -> np.ndarray:
    """Single-token softmax attention in float64 for the rows of q sharing one KV head.

    q [G, Dk], K [N, Dk], V [N, Dv] -> [G, Dv];  s = scale * q K^T,
    p = exp(s - max s), out = p V / sum p  (Thin Keys section 2; HeadQ 2.1).
    """
    q = np.asarray(q, dtype=np.float64)
    s = np.float64(scale) * (q @ np.asarray(K, dtype=np.float64).T)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return (p @ np.asarray(V, dtype=np.float64)) / p.sum(axis=-1, keepdims=True)


def rotate_query(q: np.ndarray) -> np.ndarray:
    """The key rotation applied to a query, in float64: H q / sqrt(n) with H the
    Sylvester Hadamard matrix (entry (i, j) = (-1)^popcount(i & j)), so that
    (H q) . (H k) = n q . k and the rotated scores equal the plain ones."""
    q = np.asarray(q, dtype=np.float64)
    n = q.shape[-1]
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    par = np.zeros_like(bits)
    while bits.any():
        par ^= bits & 1
        bits >>= 1
    H = np.where(par == 1, -1.0, 1.0)
    return q @ H.T / np.sqrt(n)


def decode_slab(q_group, p, q_dtype: str, k_bits: int, v_bits: int, scale,
                key_rotation: bool = False) -> np.ndarray:
    """Decode attention of the G query heads of one KV head over its packed slab
    (with key_rotation the packed keys are rotated, so the query is rotated too)."""
    Khat, Vhat = dequant_slab(p, k_bits, v_bits)
    q = upcast(q_group, q_dtype)
    if key_rotation:
        q = rotate_query(q)
    return attention(q, Khat, Vhat, scale)


def decode_all(q, packed, w, scale=None) -> np.ndarray:
    """q [B, Hq, Dk] (storage dtype) over a pack_all cache -> out float64 [B, Hq, Dv].
    Query head i reads KV head i // (Hq / Hkv)."""
    if scale is None:
        scale = default_scale(w.Dk)
    G = w.Hq // w.Hkv
    out = np.empty((w.B, w.Hq, w.Dv), dtype=np.float64)
    for b in range(w.B):
        for h in range(w.Hkv):
            p = {key: packed[key][b, h] for key in CACHE_KEYS}
            out[b, h * G:(h + 1) * G] = decode_slab(q[b, h * G:(h + 1) * G], p, w.dtype,
                                                    w.k_bits, w.v_bits, scale,
                                                    getattr(w, "key_rotation", False))
    return out


def slab_of(packed, b: int, h: int):
    return {key: packed[key][b, h] for key in CACHE_KEYS}
