"""CPU oracle of the streaming cache: one decode-time token appended at a time.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library never
calls it, and it shares no code, constant or table with the HIP library.

Source: "LogQuant: Log-Distributed 2-Bit Quantization of KV Cache" (technical
summary, section 2 "log-based filtering strategy", its dynamic adjustment: as new
tokens arrive the density of the earlier windows is halved, so tokens leave the
full-precision set at regular intervals; section 4: the order of the cached tokens
does not change attention, so full-precision and quantized tokens may be
concatenated in any order).  The pages do not spell out the per-step bookkeeping;
the readings taken here:

* retention at t tokens is ``retained_mask(t, n_recent, log_window)`` of the
  one-shot cache (positions are absolute, so every multiple of 2^j in a span keeps
  its status while the span moves forward); a token, once it has left the set, never
  comes back (true whenever log_window == 0 or n_recent >= log_window, which a
  stream requires);
* a new token is stored in fp16 (round to nearest even), like every retained token;
* a token that leaves the retained set becomes *pending*: it stays in fp16 and is
  attended as such until 32 tokens are pending; then the 32 pending tokens of
  lowest position form one group, in ascending position, quantized from their fp16
  values exactly like a group of the one-shot cache (keys per channel, values per
  token and 32-channel group) and appended after the groups packed so far;
* decode attends over every packed group and every fp16 token (retained or
  pending);
* with key rotation ("Quantize What Counts", rotation integration; the transform
  read as ``hadamard_rotate``, as for the one-shot cache) a new token's key row is
  rotated in float32 before its fp16 rounding, so the fp16 rows and the groups
  formed from them hold rotated keys, and decode rotates the query.

State of one (batch row, kv head) slab, all host NumPy:
  t              tokens appended so far (positions 0 .. t-1)
  rows           dict position -> (k fp16 bits [Dk], v fp16 bits [Dv])
  pending        set of positions in ``rows`` that have left the retained set
  groups         list of dicts, in packing order: "pos" (32 positions, ascending),
                 "k_codes" u32 [32, Dk*kb/32], "k_scale"/"k_zero" u16 [Dk],
                 "v_codes" u32 [Dv*vb], "v_scale"/"v_zero" u16 [Dv/32, 32]
"""

import numpy as np

from .kvq_oracle import (CACHE_KEYS, GROUP, attention, dequant_slab, hadamard_rotate, pack_codes, pack_slab,
                         pack_value_codes, quantize_groups, retained_mask, rotate_query, split_positions,
                         upcast)


class SlabStream:
    """Streaming cache of one slab (see the module header for the state)."""

    def __init__(self, Dk: int, Dv: int, k_bits: int, v_bits: int, n_recent: int, log_window: int,
                 v_group: int = GROUP, key_rotation: bool = False):
        if log_window > 0 and n_recent < log_window:
            raise ValueError("a stream needs log_window == 0 or n_recent >= log_window "
                             "(otherwise a token could re-enter the fp16 set)")
        self.Dk, self.Dv = Dk, Dv
        self.k_bits, self.v_bits = k_bits, v_bits
        self.n_recent, self.log_window = n_recent, log_window
        self.v_group = v_group
        self.key_rotation = key_rotation
        self.t = 0
        self.rows = {}
        self.pending = set()
        self.groups = []

    # -------------------------------------------------------------------- building
    def prefill(self, K, V, dtype: str):
        """Start the stream from the one-shot cache of T0 = len(K) tokens (``pack_slab``;
        its quantized count must be a multiple of 32).  Group g holds the compacted
        tokens 32g .. 32g+31 as in the one-shot cache; nothing is pending."""
        if self.t:
            raise ValueError("prefill starts an empty stream")
        T0 = K.shape[0]
        p = pack_slab(K, V, dtype, self.k_bits, self.v_bits, self.n_recent, self.log_window,
                      key_rotation=self.key_rotation, v_group=self.v_group)
        r, u = split_positions(T0, self.n_recent, self.log_window)
        for g in range(len(u) // GROUP):
            sl = slice(GROUP * g, GROUP * (g + 1))
            self.groups.append({
                "pos": u[sl].copy(),
                "k_codes": p["k_codes"][sl].copy(),
                "k_scale": p["k_scale"][g].copy(),
                "k_zero": p["k_zero"][g].copy(),
                "v_codes": p["v_codes"][g].copy(),
                "v_scale": p["v_scale"][g].copy(),
                "v_zero": p["v_zero"][g].copy(),
            })
        for i, pos in enumerate(r):
            self.rows[int(pos)] = (p["k_fp16"][i].copy(), p["v_fp16"][i].copy())
        self.t = T0

    def append(self, k_row, v_row, dtype: str):
        """Append the token at position t (k_row [Dk], v_row [Dv] in storage dtype).

        1. store it in fp16;  2. every stored token that is no longer retained at
        t + 1 tokens becomes pending;  3. while 32 or more are pending, the 32 of
        lowest position become the next group."""
        k32 = upcast(k_row, dtype)
        if self.key_rotation:
            k32 = hadamard_rotate(k32)
        k16 = k32.astype(np.float16).view(np.uint16)
        v16 = upcast(v_row, dtype).astype(np.float16).view(np.uint16)
        self.rows[self.t] = (k16, v16)
        self.t += 1
        keep = retained_mask(self.t, self.n_recent, self.log_window)
        for pos in self.rows:
            if not keep[pos]:
                self.pending.add(pos)
        # the fp16 set is exactly the retained set (so a packed token is never retained again)
        in_fp16 = np.zeros(self.t, dtype=bool)
        in_fp16[[pos for pos in self.rows if pos not in self.pending]] = True
        assert np.array_equal(keep, in_fp16)
        while len(self.pending) >= GROUP:
            members = sorted(self.pending)[:GROUP]
            self._pack_group(np.array(members, dtype=np.int64))

    def _pack_group(self, members):
        """Quantize the fp16 tokens ``members`` (ascending) as one group."""
        K32 = np.stack([self.rows[int(p)][0] for p in members]).view(np.float16).astype(np.float32)
        V32 = np.stack([self.rows[int(p)][1] for p in members]).view(np.float16).astype(np.float32)
        kc, ks, kz = quantize_groups(K32.T, self.k_bits)                  # [Dk, 32], [Dk]
        vc, vs, vz = quantize_groups(V32.reshape(GROUP, self.Dv // self.v_group, self.v_group), self.v_bits)
        self.groups.append({
            "pos": members.copy(),
            "k_codes": pack_codes(kc.T, self.k_bits),                      # [32, Dk*kb/32]
            "k_scale": ks.view(np.uint16),
            "k_zero": kz.view(np.uint16),
            "v_codes": pack_value_codes(vc.reshape(GROUP, self.Dv), self.v_bits),
            "v_scale": np.ascontiguousarray(vs.T).view(np.uint16),         # [Dv/gV, 32]
            "v_zero": np.ascontiguousarray(vz.T).view(np.uint16),
        })
        for p in members:
            del self.rows[int(p)]
            self.pending.discard(int(p))

    # --------------------------------------------------------------------- reading
    def as_packed(self):
        """The state as one packed slab: the groups in packing order, then the fp16
        rows in ascending position (the layout ``dequant_slab`` reads), plus the
        positions of each part."""
        nG = len(self.groups)
        words_k = self.Dk * self.k_bits // 32
        rpos = np.array(sorted(self.rows), dtype=np.int64)
        p = {
            "k_codes": (np.concatenate([g["k_codes"] for g in self.groups]) if nG
                        else np.zeros((0, words_k), np.uint32)),
            "k_scale": np.array([g["k_scale"] for g in self.groups], np.uint16).reshape(nG, self.Dk),
            "k_zero": np.array([g["k_zero"] for g in self.groups], np.uint16).reshape(nG, self.Dk),
            "v_codes": np.array([g["v_codes"] for g in self.groups], np.uint32).reshape(nG, self.Dv * self.v_bits),
            "v_scale": np.array([g["v_scale"] for g in self.groups], np.uint16).reshape(nG, self.Dv // self.v_group, GROUP),
            "v_zero": np.array([g["v_zero"] for g in self.groups], np.uint16).reshape(nG, self.Dv // self.v_group, GROUP),
            "k_fp16": np.array([self.rows[int(q)][0] for q in rpos], np.uint16).reshape(len(rpos), self.Dk),
            "v_fp16": np.array([self.rows[int(q)][1] for q in rpos], np.uint16).reshape(len(rpos), self.Dv),
        }
        group_pos = (np.concatenate([g["pos"] for g in self.groups]) if nG else np.zeros(0, np.int64))
        return p, group_pos, rpos

    def decode(self, q_group, q_dtype: str, scale) -> np.ndarray:
        """Decode attention of the G query heads of this slab's KV head over every
        token in the stream (float64; LogQuant section 4: order-free)."""
        p, _, _ = self.as_packed()
        Khat, Vhat = dequant_slab(p, self.k_bits, self.v_bits)
        q = upcast(q_group, q_dtype)
        if self.key_rotation:
            q = rotate_query(q)
        return attention(q, Khat, Vhat, scale)


def stream_keys():
    """Names of the packed arrays of ``SlabStream.as_packed`` (those of a one-shot cache)."""
    return CACHE_KEYS
