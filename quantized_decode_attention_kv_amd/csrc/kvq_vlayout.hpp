// Bit layout of the packed value codes (a library format choice).
//
// The codes of one 32-token group form a little-endian bit stream of 32*Dv*vb
// bits, i.e. Dv*vb 32-bit words (bit i of the stream is bit i%32 of word i/32).
// Channel c = 16t + n is column n of 16-channel tile t; token 8o + j of the group is
// token j of octet o.  Tokens j and j + 4 of an octet form a pair.  For every
// (octet o, column n, pair j % 4) the stream holds one field of F = Dv*vb/8 bits,
// at field index (16o + n)*4 + j%4.  A field is a run of chunks of up to
// TPW = 16/vb tiles: the chunk's r tiles' codes of the first token of the pair,
// tile by tile, then those of the second token.  Full chunks are 32 bits, so when
// Dv*vb is a multiple of 256 every chunk is one aligned word whose low half belongs
// to token j and high half to token j + 4, with tile (chunk*TPW + k) at bit k*vb
// of each half.  Masking such a word with (2^vb - 1) * 0x00010001 << k*vb gives two
// 16-bit lanes holding code * 2^(k*vb): two fp16 subnormals, one per token.
//
// Codes never straddle a word: every field and chunk starts at a multiple of vb.
//
// 3-bit codes (32 is not a multiple of 3) use a plain token-major stream instead:
// token tau, channel c at bit 3*(tau*Dv + c), so a code may straddle two words
// (stream_code reads it).  Key rows of 3-bit codes are streams too: channel c at
// bit 3c of the row.
#pragma once

#include <stdint.h>

namespace kvq {

struct ValueCodeSpot {
  int tau;  // token in the group, 0..31
  int c;    // channel
};

// bit offset of (token tau of the group, channel c) in the group's stream
__host__ __device__ inline int value_bit_position(int tau, int c, int Dv, int vb) {
  if (vb == 3) return 3 * (tau * Dv + c);
  const int n_tiles = Dv / 16, per_chunk = 16 / vb, field = Dv * vb / 8;
  const int octet = tau >> 3, j = tau & 7;
  const int tile = c >> 4, col = c & 15;
  const int chunk = tile / per_chunk, slot = tile - chunk * per_chunk;
  const int in_chunk = n_tiles - chunk * per_chunk < per_chunk ? n_tiles - chunk * per_chunk : per_chunk;
  return ((octet * 16 + col) * 4 + (j & 3)) * field + chunk * 32 + (j >> 2) * in_chunk * vb + slot * vb;
}

// inverse: which (token, channel) code sits at stream bit `bit` (a multiple of vb)
__host__ __device__ inline ValueCodeSpot value_code_at(int bit, int Dv, int vb) {
  if (vb == 3) return ValueCodeSpot{bit / 3 / Dv, bit / 3 % Dv};
  const int n_tiles = Dv / 16, per_chunk = 16 / vb, field = Dv * vb / 8;
  const int f = bit / field, within = bit - f * field;
  const int octet = f >> 6, col = (f >> 2) & 15, pair = f & 3;
  const int chunk = within >> 5, inner = within & 31;
  const int in_chunk = n_tiles - chunk * per_chunk < per_chunk ? n_tiles - chunk * per_chunk : per_chunk;
  const int upper = inner / (in_chunk * vb);
  const int slot = (inner - upper * in_chunk * vb) / vb;
  return ValueCodeSpot{octet * 8 + pair + 4 * upper, (chunk * per_chunk + slot) * 16 + col};
}

// the vb-bit code at stream bit `bit` of little-endian words w (the next word is
// read only when the code straddles into it, which only 3-bit codes do)
__host__ __device__ inline uint32_t stream_code(const uint32_t* w, int bit, int vb) {
  const int sh = bit & 31;
  uint32_t v = w[bit >> 5] >> sh;
  if (sh + vb > 32) v |= w[(bit >> 5) + 1] << (32 - sh);
  return v & ((1u << vb) - 1u);
}

}  // namespace kvq
