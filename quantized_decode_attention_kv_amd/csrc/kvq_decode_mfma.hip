// kv_decode_attn, matrix-core kernel for gfx950: four query heads per KV head,
// value head width 128.
//
// Same computation as the generic kernel (single-token decode attention read
// straight from the packed cache, see kvq_decode_generic.hip), arranged so both
// dot products run on v_mfma_f32_16x16x32_f16 and the vector ALUs do as little as
// possible per 32-token key group.
//
// Codes enter the MFMA unconverted: a code n in the low bits of an fp16 lane is
// the subnormal n * 2^-24, exactly.  A field masked in place (code times 2^k) is
// exact too as long as it stays inside the 10 mantissa bits; the 2^k is undone on
// the other operand (keys: the query operand is divided by it) or on the
// accumulator (values: every 16-channel value tile takes its codes from one bit
// slot, so the whole tile is scaled by 2^-k at the end; slots that reach past bit
// 9 are first shifted down by 8).
// Per-channel key scales and per-token value scales are folded into the other
// operand and the zero points become separate terms:
//   scores  s_t = sum_c (q_c s_c) n_tc + sum_c q_c z_c   (s_c, z_c of the key group
//           of 32, 64 or 128 tokens that holds the 32-token code group)
//   values  o_c = sum_t (p_t s_t,g) n_tc + sum_t p_t z_t,g   (g = value group of c:
//           32, 64 or 128 channels)
// The folded operands q_c s_c and p_t s_t,g are split into fp16 hi + lo parts
// (each rounded to nearest, about 22 significant bits together).
//
// Work units: one wave per unit, four independent waves per workgroup (one on
// each SIMD of a compute unit, see kWavesPerGroup); a split-K partition is one
// unit or is cut into 2, 4 or 8 (see decode_mfma_units).  The four waves of a
// workgroup form a team that shares one run of key groups of one (batch, kv head)
// slab, wave w taking every fourth group from w (see Teams below); the run starts
// come from the host with the launch.  Units share nothing until their last step: each
// stages its groups through an LDS ring of D = 2 or 3 slots (buffer loads straight
// into LDS, so up to D - 1 later groups are in flight while one is computed) and
// keeps its own online-softmax state; at the end the four units of a team combine
// their states (one barrier) and the team writes one partial result per query
// head (a unit that is a team of its own writes its own).  The launcher takes
// D = 3 where the grid puts at most 2 waves on a SIMD and its LDS keeps the whole
// grid resident, else 2 (the 128K- and 32K-token workloads: 16 waves per compute
// unit on a 2-deep ring).  Per group:
//   1. Q' = q s (hi, lo) for 64 (query, 8-channel block) tasks, one per lane, into
//      a wave-private LDS tile;
//   2. scores S^T[token, column] = codes (A: 16 tokens x 32 channels) x Q' (B), two
//      16-token tiles.  Columns 4i..4i+3 hold query i, the even ones the hi part
//      of Q', the odd ones the lo part, so one pass over the channels gives both
//      parts and every lane holds one part of the scores of one query; tile rows
//      are ordered so that lane group j holds tokens 8j..8j+7;
//   3. the key zero-point term sum_c q_c z_c: each Q' lane forms the partial sum
//      of its block, and the 16 partial sums of a query are added across lanes
//      (two exchanges inside quads, two half swaps) in fp32;
//   4. online softmax in the log2 domain: each lane of a quad adds the two parts
//      of 2 of its octet's 8 scores (DPP exchange with the neighbouring column),
//      exponentiates them and the quad shares the results (DPP broadcasts); the
//      running maximum of a query only moves (and the state is rescaled) when a
//      score exceeds it by more than 2^kHeadroom, so most groups skip the rescale;
//   5. P' = p s (hi, lo) for 64 (query, channel group, 8-token octet) tasks, again
//      one per lane and already holding the probabilities they need, into LDS;
//   6. values O[(query, part), channel] += P' (A) x codes (B), eight 16-channel
//      tiles.  A lane's B operand for tile t is its code word of that tile's
//      chunk masked to the tile's bit slot: one AND per operand register (plus
//      one shift per word for the slots above the mantissa).
// Retained fp16 rows (recent window, log-spaced tokens) join the same online state
// after the key groups: scores on the MFMA (A = fp16 key rows), values on the VALU.
// With key rotation (KVQ_KEY_ROTATION) the lane's query task is rotated before
// step 1, so the scores are those of the rotated cache.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_decode_common.hpp"
#include "kvq_internal.hpp"
#include "kvq_rotate.hpp"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kG = 4;  // query heads per KV head handled here


// log2 of the headroom a score may exceed its query's reference maximum by before
// the state is rescaled: probabilities stay <= 2^kHeadroom, so p * s stays inside
// fp16 while value scales are below 65504 / 2^kHeadroom.
constexpr int kHeadroom = 4;

// Order LDS traffic of one wave: wait for its outstanding LDS operations; the
// memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Order LDS accesses of one wave without waiting: the LDS unit executes a wave's
// ds_ operations in issue order, so a read issued after a write (or a write
// after a read) of the same wave sees the right data; only the compiler must not
// move the accesses across (it would, between lanes' different addresses).
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                0, 0);
}

// Reinterpret a packed fp16 pair.  Takes its argument by value: clang's
// __builtin_bit_cast applied directly to an element of an ext_vector_type lvalue
// reads element 0 whatever the index.
__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------- LDS staging of loads
// buffer_load ... lds: each active lane copies `bytes` (4 or 16) from
// base + voffset + soffset to lds + lane * bytes, without passing through VGPRs.
// The base sits in a buffer resource (scalar registers), the per-lane offset is
// loop-invariant and the group offset is scalar, so staging a group costs no
// vector instructions.  The wave counts the copy in vmcnt; the compiler does not
// relate it to later LDS reads, so every read of staged data follows an
// explicit wait_vmcnt.
typedef __attribute__((address_space(3))) void lds_void;
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
// raw buffer over [base, base + bytes): 32-bit dword format (gfx9 family).  Loads
// past the end return zeros without touching memory, so bytes = 0 turns every
// copy from the buffer into a no-op.
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// The copies carry the non-temporal hint (cache policy nt): every byte of the
// cache is read once per call, and the hint lets the memory hierarchy stream it
// instead of keeping it.  Measured on the 128K-token workload: 100.2 -> 92.7 us
// (kernel p50, interleaved with the plain copies on one box), 32K-token workload
// 168.8 -> 161.6 us; adding sc1 (device scope) changes nothing, sc1 alone is
// as slow as the plain copies.
constexpr int kStreamPolicy = 2;  // nt
template <int BYTES>
__device__ __forceinline__ void lds_dma(buf_rsrc r, uint32_t voffset, uint32_t soffset, void* lds) {
  static_assert(BYTES == 4 || BYTES == 16, "copy size");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voffset, soffset, 0, kStreamPolicy);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voffset, soffset, 0, kStreamPolicy);
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `ahead` (0..A) later steps of PER copies each are in
// flight: the counter bound must be an immediate, so the cases are spelled out.
template <int PER, int A>
__device__ __forceinline__ void wait_steps_ahead(int ahead) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= A)
      wait_vmcnt<PER * A>();
    else
      wait_steps_ahead<PER, A - 1>(ahead);
  }
}

// ---------------------------------------------------------------- fp16 hi/lo split
// v_fma_mix{lo,hi}_f16: fp32 fma of an fp32 and an fp16 (half H of a packed pair),
// rounded to fp16 and written to the low / high half of the destination.
template <int H>
__device__ __forceinline__ uint32_t mix_lo(float a, uint32_t b) {
  uint32_t d;
  if constexpr (H == 0)
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(b));
  else
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
template <int H>
__device__ __forceinline__ void mix_hi(uint32_t& d, float a, uint32_t b) {
  if constexpr (H == 0)
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(d) : "v"(a), "v"(b));
  else
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(d) : "v"(a), "v"(b));
}
// the same with the fp16 in half HC of c subtracted: a * b - c, one rounding
template <int H, int HC>
__device__ __forceinline__ uint32_t mix_lo_sub(float a, uint32_t b, uint32_t c) {
  uint32_t d;
  if constexpr (H == 0 && HC == 0)
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  else if constexpr (H == 1 && HC == 0)
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,1,0] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  else if constexpr (H == 0 && HC == 1)
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  else
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}
template <int H, int HC>
__device__ __forceinline__ void mix_hi_sub(uint32_t& d, float a, uint32_t b, uint32_t c) {
  if constexpr (H == 0 && HC == 0)
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(b), "v"(c));
  else if constexpr (H == 1 && HC == 0)
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,1,0] op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(b), "v"(c));
  else if constexpr (H == 0 && HC == 1)
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(b), "v"(c));
  else
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "+v"(d) : "v"(a), "v"(b), "v"(c));
}

// x[k] * s_k for k = 0..7 (s: 8 fp16 in natural order, s_k in half k%2 of dword
// k/2) as hi + lo fp16 parts; operand dword m pairs elements m and m + 4.
template <int M>
__device__ __forceinline__ void split_pair(const float (&x)[8], const u32x4& s, u32x4& hi, u32x4& lo) {
  constexpr int H = M & 1;
  uint32_t h = mix_lo<H>(x[M], s[M >> 1]);
  mix_hi<H>(h, x[M + 4], s[(M >> 1) + 2]);
  uint32_t l = mix_lo_sub<H, 0>(x[M], s[M >> 1], h);
  mix_hi_sub<H, 1>(l, x[M + 4], s[(M >> 1) + 2], h);
  hi[M] = h;
  lo[M] = l;
}
__device__ __forceinline__ void split8(const float (&x)[8], const u32x4& s, u32x4& hi, u32x4& lo) {
  split_pair<0>(x, s, hi, lo);
  split_pair<1>(x, s, hi, lo);
  split_pair<2>(x, s, hi, lo);
  split_pair<3>(x, s, hi, lo);
}

// ------------------------------------------------------------------ key codes
// 8 codes of one 8-channel block -> 4 operand dwords, dword m = codes (m, m+4),
// fields masked in place: dword m carries the codes times key_code_scale(m).
template <int BITS>
__host__ __device__ constexpr float key_code_scale(int m) {
  return BITS == 2 ? float(1 << (2 * m)) : (BITS == 4 ? ((m & 1) ? 16.0f : 1.0f) : 1.0f);
}
__device__ __forceinline__ u32x4 keys2(uint32_t w, int hi) {
  const uint32_t y = __builtin_amdgcn_perm(w, w, hi ? 0x0C030C02u : 0x0C010C00u);
  return u32x4{y & 0x00030003u, y & 0x000C000Cu, y & 0x00300030u, y & 0x00C000C0u};
}
__device__ __forceinline__ u32x4 keys4(uint32_t w) {
  const uint32_t w8 = w >> 8;
  return u32x4{w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
}
__device__ __forceinline__ u32x4 keys8(uint32_t lo, uint32_t hi) {
  u32x4 d;
#pragma unroll
  for (int m = 0; m < 4; ++m) d[m] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + uint32_t(m) * 0x00010001u);
  return d;
}
template <int BITS, int NW>
__device__ __forceinline__ u32x4 key_field(const uint32_t (&w)[NW], int idx) {
  if constexpr (BITS == 2) return keys2(w[idx >> 1], idx & 1);
  else if constexpr (BITS == 4) return keys4(w[idx]);
  else return keys8(w[2 * idx], w[2 * idx + 1]);
}

// ---------------------------------------------------------------- value codes
// Bit position, inside each 16-bit half of a code word, at which the codes of the
// tile in slot `slot` enter the MFMA: the slot's own position slot*VB while the
// field ends inside the mantissa (bit 9), else 8 lower (the word is shifted right
// by 8 first; codes of the upper half stay in the upper half).
template <int VB>
__host__ __device__ constexpr int value_tile_shift(int slot) {
  return slot * VB + VB <= 10 ? slot * VB : slot * VB - 8;
}

template <int NB>  // load NB bytes (2, 4, 8, 16 or 32) into words
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t (&w)[NB < 4 ? 1 : NB / 4]) {
  if constexpr (NB == 2) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (NB == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NB == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < NB / 16; ++k) {
      const u32x4 v = reinterpret_cast<const u32x4*>(p)[k];
      w[4 * k] = v[0];
      w[4 * k + 1] = v[1];
      w[4 * k + 2] = v[2];
      w[4 * k + 3] = v[3];
    }
  }
}

// LDS of one wave, in bytes (at most 20 KB for the common shapes, 10 KB or less
// where 16 waves share a compute unit):
//   a ring of D slots (D key groups in flight), one key group each: key codes,
//   value codes, key scales, key zeros, value scales, value zeros;
//   the Q' operand tile of the group being computed (KK chunks of 32 channels)
//   and its P' operand tile, which shares the Q' tile's bytes when it fits there
//   (the Q' operands are consumed before P' is written).  With D > 2 the tiles
//   sit in the group's own slot, which is idle once the group has been read into
//   registers (it is refilled one step later); with D == 2 the slot is refilled
//   at once, so the tiles have an area of their own.
//   After the loop the ring holds the q hi/lo operand B2 of the retained rows
//   (slot 0) and their probabilities PT (slot 1), then the matrix-core output
//   and the value zero-point sums.
// P' tiles of the ring instances: the entries of channel group gc start at
// gc * kPASkew (16-byte entries, see the kernel)
constexpr int kPASkew = 36;
template <int DK, int DV, int KB, int VB, int D>
struct Lds {
  static constexpr int KK = DK / 32, NGV = DV / 32;
  static constexpr bool kInSlot = D > 2;
  static constexpr int kQB1 = KK * 32 * 16;   // one Q' tile
  static constexpr int kPA1 = (kInSlot ? (NGV - 1) * kPASkew + 32 : NGV * 32) * 16;  // one P' tile
  static constexpr int kStK = 32 * DK * KB / 8;
  static constexpr int kStV = 32 * DV * VB / 8;
  static constexpr int kStS = 256;
  static constexpr int kStage = kStK + kStV + 4 * kStS;
  // the P' tile of a group is written after its Q' tile has been read, so the two
  // can share one area (ring instances; with D == 2 they share it only when the
  // P' tile is not the larger, which keeps those instances' occupancy)
  static constexpr bool kShare = kInSlot || kPA1 <= kQB1;
  static constexpr int kTiles = kShare ? (kPA1 > kQB1 ? kPA1 : kQB1) : kQB1 + kPA1;
  static constexpr int kPAOff = kShare ? 0 : kQB1;
  static constexpr int kSlot = kInSlot && kTiles > kStage ? kTiles : kStage;
  static constexpr int kSlots = D;
  static constexpr int oTiles = kInSlot ? 0 : kSlots * kSlot;  // separate tile area (D == 2)
  static constexpr int kBytes = kSlots * kSlot + (kInSlot ? 0 : kTiles);
  static_assert(kQB1 <= kSlot && kG * 32 * 4 <= kSlot && kG * (DV + NGV) * 4 <= kSlots * kSlot, "aliases");
};

// v from lane j' of each quad of lanes (quad_perm broadcast: all four lanes of a
// quad read lane j')
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), J * 0x55, 0xF, 0xF, true));
}
// v of lane l ^ 1 and of lane l ^ 2 (quad_perm 1,0,3,2 and 2,3,0,1; every source
// lane exists, and bound_ctrl lets the compiler fold the move into the ALU
// operation that consumes it)
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
// op over the four lanes of each quad (two exchanges: lanes l ^ 1, then l ^ 2)
template <bool MAX>
__device__ __forceinline__ float quad_allreduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, quad_xor1(v));
  return op(v, quad_xor2(v));
}
// Sum (or max) of v over the 16 lanes l with (l / 4) % 4 == (lane / 4) % 4: the
// quad, then the two gfx950 half swaps across rows.  Every step pairs lanes
// symmetrically, so all 16 lanes end with the same bits.
template <bool MAX>
__device__ __forceinline__ float query_allreduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = quad_allreduce<MAX>(v);
  const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(h32[0]), __uint_as_float(h32[1]));
  const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(h16[0]), __uint_as_float(h16[1]));
}

// Work units.  A unit is one wave; a team is TS units (4, one workgroup, or 1)
// that share a contiguous run of key groups of one (batch, kv head) slab.  Units
// are independent until the epilogue, where a team of 4 combines its units'
// states after one barrier and writes one partial result.
//
// First key group of team t of T over nG groups, for R waves per SIMD.  The
// workgroup dispatcher fills the SIMDs round-robin in grid order, so with the
// team-major grid and one team per resident workgroup the teams t < T/R become
// the oldest waves on their SIMDs, the next T/R the second oldest, and so on;
// waves are served oldest first, so run lengths fall by rank (integer weights
// 100 + s (R - 1 - 2 r) for rank r, s = span / (R - 1): with 2 waves per SIMD
// span 16, the oldest and youngest rank differing by +-16%, measured on the 128K
// workload (then on 2048 waves) to bring the finish times of the two waves of a
// SIMD within a few microseconds, and slower on the 16K workload with 28; with 3
// or 4 waves per SIMD span 28 (128K workload on 4096 waves: 93.3 -> 91.5 and
// 97.9 -> 96.2 us p50 inside the step on two boxes, interleaved)).
// Retained fp16 rows come in 32-row tiles; unit u takes tiles u, u + U, ..., so
// the waves of a team take the same number of tiles (tq, plus one in the first
// ceil(tm / TS) teams, tm = tiles % U), and a team's run is shortened by what its
// waves spend on tiles: teams share nG plus the tiles' cost (tc16 sixteenths of a
// group per tile and wave) by rank weight, less their own tiles' cost.  The
// cost is capped so that every team keeps at least one group, which keeps the
// starts increasing.  Any split gives the same result up to rounding.
__host__ __device__ inline int team_start(int t, int T, int TS, int nG, int R, int tq, int tm, int tc16) {
  const int64_t s = R > 1 ? (R > 2 ? 28 : 16) / (R - 1) : 0;
  int64_t wb = 0, wall = 0;
  for (int r = 0; r < R; ++r) {
    const int64_t lo = (int64_t(r) * T + R - 1) / R, hi = (int64_t(r + 1) * T + R - 1) / R;  // teams of rank r
    const int64_t w = 100 + s * (R - 1 - 2 * r);
    wall += w * (hi - lo);
    wb += w * (t < lo ? 0 : (t < hi ? t - lo : hi - lo));
  }
  const int64_t tmt = (tm + TS - 1) / TS;            // teams whose waves take tq + 1 tiles
  const int64_t emax = tq + (tmt > 0 ? 1 : 0);       // most tiles a wave takes
  int64_t c = tc16;
  if (emax > 0) {
    // every team's share stays >= 1 group: 16 nG wmin / wall - TS c emax >= 16
    const int64_t wmin = 100 - s * (R - 1);
    const int64_t room = (16 * int64_t(nG) * wmin) / wall - 16;
    c = room > 0 ? (c < room / (int64_t(TS) * emax) ? c : room / (int64_t(TS) * emax)) : 0;
  }
  const int64_t e_before = int64_t(t) * tq + (int64_t(t) < tmt ? int64_t(t) : tmt);
  const int64_t e_all = int64_t(T) * tq + (int64_t(T) < tmt ? int64_t(T) : tmt);
  const int64_t w16 = 16 * int64_t(nG) + int64_t(TS) * c * e_all;
  const int64_t st16 = w16 * wb / wall - int64_t(TS) * c * e_before;
  const int64_t g = st16 / 16;
  return int(g < 0 ? 0 : (g > nG ? int64_t(nG) : g));
}

// Cost of a retained 32-row tile in sixteenths of a key group's time (measured:
// about 2.5 groups' time where a tile is 4 groups' bytes, so 5/8 of the byte ratio).
template <int DK, int DV, int KB, int VB>
__host__ __device__ inline int tile_cost16(const kvq_layout& L) {
  constexpr int64_t kTileBytes = 32 * (DK + DV) * 2;
  const int64_t group_bytes = 32 * (DK * KB + DV * VB) / 8 + ((DK * 4) >> (L.k_group == 128 ? 2 : (L.k_group == 64 ? 1 : 0))) +
                              ((DV / 32 * 32 * 4) >> (L.v_group == 128 ? 2 : (L.v_group == 64 ? 1 : 0)));
  return int(16 * 5 * kTileBytes / (8 * group_bytes));
}

// Waves per SIMD that the LDS of one unit allows on a 160 KB compute unit (at most
// 4, which is the 16 waves per CU of the common shapes); the register budget
// is set to match, so registers never limit occupancy below what LDS allows.
template <int DK, int DV, int KB, int VB, int D>
constexpr int lds_waves_per_simd() {
  const int per_cu = (160 * 1024) / Lds<DK, DV, KB, VB, D>::kBytes;
  return per_cu >= 16 ? 4 : (per_cu >= 4 ? per_cu / 4 : 1);
}

// Waves per workgroup.  The waves of a workgroup are independent units (no
// barriers, an LDS slice each); grouping them by four places one on each SIMD of
// a compute unit whatever state the dispatcher is in.  Single-wave workgroups were
// spread 1 / 2 / 3 per SIMD (8% of SIMDs with 3) when the decode followed the pack
// kernel, and those SIMDs finished 20 us after the rest.
constexpr int kWavesPerGroup = 4;

template <int DK, int DV, int KB, int VB, int D>
__global__ __launch_bounds__(64 * kWavesPerGroup, (lds_waves_per_simd<DK, DV, KB, VB, D>())) void decode_mfma_kernel(const DecodeArgs a) {
  using LL = Lds<DK, DV, KB, VB, D>;
  constexpr int KK = DK / 32;          // 32-channel score steps
  constexpr int NV = DV / 16;          // 16-channel value tiles
  constexpr int NGV = DV / 32;         // 32-channel value groups
  constexpr int TPW = 16 / VB;         // value tiles per code word
  constexpr int NCH = NV / TPW;        // code words per token pair
  constexpr int VLW = 4 * NCH;         // value code words per lane and group
  constexpr int KROW = DK * KB / 8;    // bytes of one key row
  constexpr int KLB = KROW / 4;        // key-row bytes per lane (a quarter row)
  constexpr int KLW = KLB < 4 ? 1 : KLB / 4;
  constexpr uint32_t kVMask = ((1u << VB) - 1u) * 0x00010001u;
  static_assert(DV == 128 && NV % TPW == 0 && KLB >= 4 && DK % 32 == 0 && DK <= 128, "shape");

  extern __shared__ __align__(16) unsigned char lds_all[];
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);  // uniform in the wave
  unsigned char* const smem = lds_all + wave * LL::kBytes;      // this wave's slice
  unsigned char* stage = smem;                                 // [D][kSlot]
  u32x4* B2 = reinterpret_cast<u32x4*>(smem);                  // q hi/lo, retained rows
  float* PT = reinterpret_cast<float*>(smem + LL::kSlot);      // [4][32], retained rows
  const int lane = int(threadIdx.x) & 63, n = lane & 15, gq = lane >> 4;

  // Teams.  When the unit count is a multiple of 4, the 4 waves of a workgroup are
  // the 4 units of one team, which shares one run of key groups of one slab: wave w
  // takes groups first + w, first + w + 4, ..., so the workgroup reads 4
  // consecutive groups at a time (measured: the memory system streams the cache
  // about 7% faster this way than as 4 separate runs).  The grid is team-major:
  // workgroup L is team L / slabs of slab L % slabs.  Otherwise each wave is a team
  // of its own and the grid is unit-major: wave L = 4 block + wave is unit L / slabs
  // of slab L % slabs (the last block may hold waves past the grid, which leave at
  // once).
  const int U = a.units, slabs = a.L.B * a.L.Hkv;
  const int TS = (U % kWavesPerGroup) == 0 ? kWavesPerGroup : 1;  // waves per team
  int team, unit, sl;
  if (TS == kWavesPerGroup) {
    team = int(blockIdx.x) / slabs;
    sl = int(blockIdx.x) % slabs;
    unit = team * kWavesPerGroup + wave;
  } else {
    const int gw = int(blockIdx.x) * kWavesPerGroup + wave;
    team = unit = gw / slabs;
    sl = gw % slabs;
  }
  if (unit >= U) return;
  const int h = sl % a.L.Hkv, b = sl / a.L.Hkv;
  const int nG = a.L.n_groups, R = a.L.R;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  // the team's run [tg0, tg1); this wave's groups are g0 + TS j, j < nj
  const int T = U / TS;
  // retained tiles: this unit takes tiles unit, unit + U, ... (tq or tq + 1 of them)
  const int nRT = (R + 31) / 32;  // 32-row tiles of retained rows
  const int tq = nRT / U, tm = nRT % U;
  // (the host passes the run starts of up to kMaxTeamTable teams with the launch:
  // computing them here would delay the first copies by a few microseconds)
  int tg0, tg1;
  if (a.n_team_first > 0) {
    tg0 = a.team_first[team];
    tg1 = a.team_first[team + 1];
  } else {
    const int tc16 = tile_cost16<DK, DV, KB, VB>(a.L);
    tg0 = team_start(team, T, TS, nG, a.ranks, tq, tm, tc16);
    tg1 = team_start(team + 1, T, TS, nG, a.ranks, tq, tm, tc16);
  }
  const int g0 = tg0 + (unit - team * TS);
  const int nj = g0 < tg1 ? (tg1 - g0 + TS - 1) / TS : 0;

  // per-slab bases (wave-uniform)
  const uint8_t* kbase = static_cast<const uint8_t*>(a.cache.k_codes) + slab * a.g_stride * (KVQ_GROUP * KROW);
  // key scales / zeros: one row of DK per key group of 32 << ksh tokens, i.e. per
  // 1 << ksh code groups (scalar register, as vsh below)
  const int ksh = __builtin_amdgcn_readfirstlane(a.L.k_group == 128 ? 2 : (a.L.k_group == 64 ? 1 : 0));
  const uint16_t* ksbase = static_cast<const uint16_t*>(a.cache.k_scale) + slab * (a.g_stride >> ksh) * DK;
  const uint16_t* kzbase = static_cast<const uint16_t*>(a.cache.k_zero) + slab * (a.g_stride >> ksh) * DK;
  const uint32_t* vbase = static_cast<const uint32_t*>(a.cache.v_codes) + slab * a.g_stride * (DV * VB);
  // value scales / zeros: (Dv / v_group) x 32 per group, v_group = 32 << vsh
  // (kept in a scalar register: the copies below take it in their descriptors)
  const int vsh = __builtin_amdgcn_readfirstlane(a.L.v_group == 128 ? 2 : (a.L.v_group == 64 ? 1 : 0));
  const uint16_t* vsbase = static_cast<const uint16_t*>(a.cache.v_scale) + slab * a.g_stride * (DV >> vsh);
  const uint16_t* vzbase = static_cast<const uint16_t*>(a.cache.v_zero) + slab * a.g_stride * (DV >> vsh);

  // Q' task of this lane: (block tb = 8-channel block kk_t of lane group gq_t,
  // query i_t); it also forms the block's key zero-point partial sum
  const int kk_t = lane >> 4, i_t = (lane >> 2) & 3, gq_t = lane & 3;
  const bool qtask = kk_t < KK;
  const int tb = gq_t * KK + (qtask ? kk_t : 0);
  // score columns: n = 4 iq + rep holds part rep % 2 (hi, lo) of query iq;
  // P' task: (query iq, channel group rep, octet gq)
  const int iq = n >> 2, rep = n & 3;
  const int gcP = rep;

  // ------------------------------------------------- staging of key groups
  // Every piece of a group is copied so that the lane that consumes it reads it
  // back from the place of its own lane id (LDS reads contiguous across the wave):
  //   key codes: per tile, KNP pieces of KPB bytes (the lane's quarter row);
  //   value codes: VLW / 4 pieces of 16 bytes (the lane's words);
  //   key scales, key zeros, value scales, value zeros: one 4-byte copy per lane
  //   each, 256 bytes per array and group (the key arrays of DK < 128 have fewer
  //   bytes; the surplus lanes read past the end of the buffer, which returns
  //   zeros into the unused part of the array's 256-byte area).
  // Every copy is a buffer load with all lanes active, so the wave's copies
  // complete in issue order and the waits below can count them.
  // Key rows of 32 bytes (8 bytes per lane and tile) are the exception: the
  // group's 1 KB of key codes is one 16-byte copy per lane (four 4-byte pieces
  // measured about 6% slower to stream).  Copy lane i = 16 (2 tt + h) + 4 j + q
  // fetches half h of row 8 j + 4 tt + q, so the lanes that read tile tt, half h
  // find their 16 rows in 16 consecutive 16-byte places (conflict-free 8-byte reads).
  constexpr int KPB = KLB >= 16 ? 16 : 4;   // bytes per key piece
  constexpr int KNP = KLB / KPB;            // key pieces per tile
  constexpr int VNP = VLW / 4;              // value pieces
  constexpr bool KLIN = KROW == 32;         // the group's key codes as one copy in memory order
  constexpr int kDmas = (KLIN ? 1 : 2 * KNP) + VNP + 4;  // copies per group
  constexpr int oKZ = LL::kStS, oVS = 2 * LL::kStS, oVZ = 3 * LL::kStS;  // scale area offsets
  static_assert(DK * 2 <= LL::kStS && DV * 2 == LL::kStS, "scale area");
  static_assert((D - 1) * kDmas < 64 && D >= 2, "vmcnt");
  static_assert(KLB % KPB == 0 && VLW % 4 == 0 && DK / 8 <= 64 && 4 * NGV <= 64, "staging");
  // per-lane byte offsets inside a group (the group base itself is wave-uniform)
  uint32_t koff[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) koff[tt] = uint32_t(8 * (n >> 2) + 4 * tt + (n & 3)) * KROW + gq * KLB;
  const uint32_t klin = uint32_t(8 * ((lane >> 2) & 3) + 4 * (lane >> 5) + (lane & 3)) * 32u + 16u * ((lane >> 4) & 1);
  const uint32_t voff = uint32_t(lane) * (VLW * 4);
  // scale copies: byte offset of this lane's dword (past the end for surplus lanes)
  const uint32_t kso = lane < DK / 2 ? uint32_t(lane) * 4 : 0x80000000u;
  const uint32_t vso = lane < ((DV / 2) >> vsh) ? uint32_t(lane) * 4 : 0x80000000u;
  // a unit without key groups gets empty buffers (its cache buffers may be null)
  const int nrec = nj > 0 ? 0x7fffffff : 0;
  const buf_rsrc rk = make_rsrc(kbase, nrec), rv = make_rsrc(vbase, nrec);
  const int nsk = nj > 0 ? (nG >> ksh) * DK * 2 : 0, nsv = nj > 0 ? nG * ((DV * 2) >> vsh) : 0;
  const buf_rsrc rks = make_rsrc(ksbase, nsk), rkz = make_rsrc(kzbase, nsk);
  const buf_rsrc rvs = make_rsrc(vsbase, nsv), rvz = make_rsrc(vzbase, nsv);
  const buf_rsrc r_none = make_rsrc(nullptr, 0);  // copies from it touch no memory
  // `live` false: the same copies from an empty buffer (counted like the others,
  // no memory traffic)
  auto stage_group = [&](int g, int slot, bool live) {
    unsigned char* sb = stage + slot * LL::kSlot;
    const uint32_t gk = uint32_t(g) * (32 * KROW);
    const buf_rsrc rk_ = live ? rk : r_none, rv_ = live ? rv : r_none;
    if constexpr (KLIN) {
      lds_dma<16>(rk_, klin, gk, sb);
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int hp = 0; hp < KNP; ++hp) lds_dma<KPB>(rk_, koff[tt] + hp * KPB, gk, sb + (tt * KNP + hp) * 64 * KPB);
      }
    }
    const uint32_t gv = uint32_t(g) * (DV * VB * 4);
#pragma unroll
    for (int k = 0; k < VNP; ++k) lds_dma<16>(rv_, voff + 16 * k, gv, sb + LL::kStK + k * 1024);
    unsigned char* ss = sb + LL::kStK + LL::kStV;
    lds_dma<4>(live ? rks : r_none, kso, uint32_t(g >> ksh) * (DK * 2), ss);
    lds_dma<4>(live ? rkz : r_none, kso, uint32_t(g >> ksh) * (DK * 2), ss + oKZ);
    lds_dma<4>(live ? rvs : r_none, vso, uint32_t(g) * uint32_t((DV * 2) >> vsh), ss + oVS);
    lds_dma<4>(live ? rvz : r_none, vso, uint32_t(g) * uint32_t((DV * 2) >> vsh), ss + oVZ);
  };
  // The query first (vector-memory operations complete in order, so it would
  // otherwise wait for the staged groups): the 8 elements of the lane's Q' task.
  // Then the groups of the first D steps into the ring (a unit with fewer groups
  // issues the rest as copies that touch no memory, so every unit has D steps'
  // copies counted).
  // Raw bytes, converted only after the copies are issued (a conversion next to
  // the load would make the wave wait for it first); the buffer spans the kG
  // query rows of this KV head, so the 32-byte read of a 16-bit query stays inside.
  const int64_t qhead = (int64_t(b) * a.L.Hq + int64_t(h) * kG) * DK;
  const int qesz = a.q_dtype == KVQ_F32 ? 4 : 2;
  const buf_rsrc rq = make_rsrc(static_cast<const uint8_t*>(a.q) + qhead * qesz, kG * DK * qesz);
  const uint32_t qoff = uint32_t(i_t * DK + 8 * tb) * uint32_t(qesz);
  const u32x4 qw0 = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, 0, 0);
  const u32x4 qw1 = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 16, 0, 0);
#pragma unroll
  for (int u = 0; u < D; ++u) stage_group(g0 + TS * u, u, u < nj);
  __builtin_amdgcn_sched_barrier(0);
  float qx[8];
  if (a.q_dtype == KVQ_BF16) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      qx[2 * d] = __uint_as_float(qw0[d] << 16);
      qx[2 * d + 1] = __uint_as_float(qw0[d] & 0xFFFF0000u);
    }
  } else if (a.q_dtype == KVQ_F16) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const half2_t hh = as_half2(qw0[d]);
      qx[2 * d] = float(hh[0]);
      qx[2 * d + 1] = float(hh[1]);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      qx[d] = __uint_as_float(qw0[d]);
      qx[4 + d] = __uint_as_float(qw1[d]);
    }
  }

  if (a.L.flags & KVQ_KEY_ROTATION) {
    // the packed keys are rotated: rotate the query the same way.  Channel
    // 8 tb + k of the task: butterflies 1, 2, 4 over k in registers, then bit s of
    // tb, which is bit s of kk_t (lane ^ 16 << s) for s < log2 KK, else bit
    // s - log2 KK of gq_t (lane ^ 1 << (s - log2 KK)); lanes without a task
    // exchange only among themselves
    constexpr int LKK = KK == 1 ? 0 : (KK == 2 ? 1 : (KK == 4 ? 2 : 3));
    static_assert((1 << LKK) == KK, "power-of-two key width");
    butterflies8(qx);
#pragma unroll
    for (int st = 0; st < LKK + 2; ++st) {
      const int pl = st < LKK ? (16 << st) : (1 << (st - LKK));
      const bool up = ((tb >> st) & 1) != 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) qx[k] = butterfly(qx[k], __shfl_xor(qx[k], pl), up);
    }
    const float sc = rotation_scale(LKK + 5);
#pragma unroll
    for (int k = 0; k < 8; ++k) qx[k] *= sc;
  }

  // ---------------------------------------------------------------- set-up
  // Query i_t is scaled by 2^-E, E >= 0 the smallest exponent such that
  // |q 2^-E| <= 1, which keeps q_c s_c inside the fp16 range; every use of the
  // exponent in this lane concerns query (lane / 4) % 4 (= i_t = iq).
  float qmax = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    qx[k] *= a.scale * kLog2e;
    qmax = fmaxf(qmax, fabsf(qx[k]));
  }
  qmax = query_allreduce<true>(qtask ? qmax : 0.0f);
  float qe;
  {
    int e = 0;
    frexpf(qmax, &e);
    qe = qmax > 1.0f ? ldexpf(1.0f, -e) : 1.0f;
  }
  // the lane's Q' task: q 2^-E divided by the code scale of each operand slot,
  // and q 2^-E itself for the zero-point partial sum
  float qsv[8], qzv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    qzv[k] = qtask ? qx[k] * qe : 0.0f;
    qsv[k] = qzv[k] * (1.0f / key_code_scale<KB>(k & 3));
  }
  // LDS tile entries (16 bytes each) are stored swizzled so that the 16 lanes of
  // each row of the wave hit 16 different 16-byte bank slots:
  //   Q' entry (kk*4 + gq)*8 + 4*part + i at e ^ (bit 4 of e) << 2 (rows 2, 3 of
  //   the 4 gq rows swap their hi and lo halves);
  //   P' entry (gc*4 + gq)*8 + j: with a ring of 3 or more at gc * kPASkew + gq*8 + j
  //   (the skew of 4 entries per channel group spreads a row's writes over 16
  //   bank slots and keeps the lane part of every address independent of gc),
  //   else at e ^ (gc & 1) << 3 ^ (gc >> 1) << 2.
  // The swizzled addresses take a few more registers: three instances held to 128
  // (the 2-deep rings of K2V4 at key widths 64 and 128 and of K8V2 at width 32,
  // 4 waves per SIMD) would spill with them and keep the plain order.  Measured
  // on the 2-deep K4V2 ring of the 128K workload: 101.1 -> 92.1 us p50 inside the
  // step, 102.9 -> 94.1 as cold calls (LDS bank-conflict cycles per LDS
  // instruction 4.8 with the plain order).
  constexpr bool kSwz = !(D == 2 && lds_waves_per_simd<DK, DV, KB, VB, D>() == 4 &&
                          ((KB == 2 && VB == 4 && DK >= 64) || (DK == 32 && KB == 8 && VB == 2)));
  auto qb_at = [](int e) { return kSwz ? e ^ (((e >> 4) & 1) << 2) : e; };
  auto pa_at = [](int e) { return kSwz ? e ^ (((e >> 5) & 1) << 3) ^ (((e >> 6) & 1) << 2) : e; };
  // place of P' entry (gc, x = gq*8 + j)
  auto pa_pos = [&](int gc, int x) { return LL::kInSlot ? gc * kPASkew + x : pa_at(gc * 32 + x); };
  // this lane's Q' read (channel block kk adds kk * 512 bytes) and P' read (any gc)
  const int qb_rd = qb_at(gq * 8 + 4 * (rep & 1) + iq) * 16;
  const int qb_entry = ((qtask ? kk_t : 0) * 4 + gq_t) * 8 + i_t;
  // Key zero-point term of query i_t: sum_c q_c z_c (times 2^-E), from the lanes'
  // 8-channel partial sums: the 16 lanes of a query are the quads 16 kk + 4 i_t,
  // so two exchanges inside each quad and two row swaps give every lane the
  // total of its query.
  auto zero_term = [&](const u32x4& kz) -> float {
    float zp = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const half2_t zz = as_half2(kz[k >> 1]);
      zp = fmaf(qzv[k], float(zz[k & 1]), zp);
    }
    return query_allreduce<false>(zp);
  };
  const float coefB = 1.0f / qe;           // q was scaled by 2^-E (query iq)
  const float coefD = 16777216.0f * coefB;  // codes are n 2^-24
  const int pa_hi = pa_pos(gcP, gq * 8 + iq) * 16, pa_lo = pa_pos(gcP, gq * 8 + iq + 4) * 16;
  const int vs_at = ((gcP >> vsh) * 4 + gq) * 16;  // the lane's 8 value scales / zeros in a slot

  // online-softmax state: reference maxima per query (wave-uniform) and this
  // lane's copy for its query; l over the lane's tokens; value accumulators
  float m_q[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i) m_q[i] = -INFINITY;
  float m_lane = -INFINITY, l_run = 0.0f, zacc = 0.0f;
  f32x4 oacc[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t) oacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float o_r[kG][2];  // retained rows (VALU): channels 2 lane, 2 lane + 1
#pragma unroll
  for (int i = 0; i < kG; ++i) o_r[i][0] = o_r[i][1] = 0.0f;

  // Softmax update of one key group (or 32-row tile of retained rows).  v = the
  // lane's raw MFMA outputs: part rep % 2 of the scores of query iq for the 8
  // tokens of octet gq (v[4 tt + r] = token 8 gq + 4 tt + r); lanes rep and
  // rep ^ 1 of a quad hold the two parts.  score = v * coef + bias (log2 domain).
  // Lane rep of the quad adds the parts of tokens 2 rep and 2 rep + 1 (those of
  // tile rep / 2, exchanged with its neighbour), exponentiates them and adds them
  // to its l; the quad shares the results, so pv returns all 8 probabilities of
  // the octet, relative to the (possibly moved) reference maximum.
  // rescale_acc(alpha) rescales the value accumulators when a reference moves.
  const bool rep_hi = (rep & 2) != 0, rep_odd = (rep & 1) != 0;
  auto softmax_step = [&](const float (&v)[8], float coef, float bias, float (&pv)[8], auto&& rescale_acc) {
    // (scalars, not an array: a select between two elements of a local array can
    // become a load through a selected address, which puts the array on the stack)
    const float m0 = rep_hi ? v[4] : v[0], m1 = rep_hi ? v[5] : v[1];
    const float m2 = rep_hi ? v[6] : v[2], m3 = rep_hi ? v[7] : v[3];
    const float f0 = quad_xor1(m0) + m0, f1 = quad_xor1(m1) + m1;
    const float f2 = quad_xor1(m2) + m2, f3 = quad_xor1(m3) + m3;
    const float x0 = rep_odd ? f2 : f0, x1 = rep_odd ? f3 : f1;
    float s0 = fmaf(x0, coef, bias - m_lane), s1 = fmaf(x1, coef, bias - m_lane);
    if (__builtin_expect(__any(fmaxf(s0, s1) > float(kHeadroom)), 0)) {
      // some score left the headroom: move those references to the group maxima
      // (the quad's maximum, then one lane per octet)
      const float b0 = fmaf(x0, coef, bias), b1 = fmaf(x1, coef, bias);
      const float mab = quad_allreduce<true>(fmaxf(b0, b1));
      float alpha[kG];
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        float mg = readlane_f32(mab, 4 * i);
#pragma unroll
        for (int j = 1; j < 4; ++j) mg = fmaxf(mg, readlane_f32(mab, 16 * j + 4 * i));
        const float m_new = mg > m_q[i] + float(kHeadroom) ? mg : m_q[i];
        alpha[i] = lse_weight(m_q[i], m_new);
        m_q[i] = m_new;
      }
      float al = alpha[0];
      m_lane = m_q[0];
#pragma unroll
      for (int i = 1; i < kG; ++i) {
        if (iq == i) {
          al = alpha[i];
          m_lane = m_q[i];
        }
      }
      l_run *= al;
      zacc *= al;
      rescale_acc(alpha);
      s0 = b0 - m_lane;
      s1 = b1 - m_lane;
    }
    const float e0 = fast_exp2(s0), e1 = fast_exp2(s1);
    l_run += e0 + e1;
    pv[0] = quad_bcast<0>(e0);
    pv[1] = quad_bcast<0>(e1);
    pv[2] = quad_bcast<1>(e0);
    pv[3] = quad_bcast<1>(e1);
    pv[4] = quad_bcast<2>(e0);
    pv[5] = quad_bcast<2>(e1);
    pv[6] = quad_bcast<3>(e0);
    pv[7] = quad_bcast<3>(e1);
  };
  auto rescale_retained = [&](const float (&alpha)[kG]) {
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      o_r[i][0] *= alpha[i];
      o_r[i][1] *= alpha[i];
    }
  };
  auto rescale_groups = [&](const float (&alpha)[kG]) {
#pragma unroll
    for (int t = 0; t < NV; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[t][r] *= alpha[r];
    }
    rescale_retained(alpha);
  };

  // ------------------------------------------------------------ key groups
  // everything one key group needs, read back from its ring slot
  struct GroupLoads {
    uint32_t kw[2][KLW];  // key codes of tiles 0, 1 (row n = token 8(n/4) + 4tt + n%4)
    uint32_t vw[VLW];     // value code words: pair m, chunk c at m*NCH + c
    u32x4 ks, kz;         // key scales / zeros of the lane's Q' block
    u32x4 vs, vz;         // value scale / zero of the lane's P' channel group, tokens 8gq..
  };
  auto read_group = [&](int slot, GroupLoads& d) {
    const unsigned char* sb = stage + slot * LL::kSlot;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if constexpr (KLIN) {
        // two 4-byte reads: with one 8-byte read the compiler cannot tell it from
        // the copies in flight and waits for all of them
        const uint32_t* src = reinterpret_cast<const uint32_t*>(sb + (32 * tt + 16 * (gq >> 1) + n) * 16 + 8 * (gq & 1));
        d.kw[tt][0] = src[0];
        d.kw[tt][1] = src[1];
      } else {
#pragma unroll
        for (int hp = 0; hp < KNP; ++hp) {
          const unsigned char* src = sb + (tt * KNP + hp) * 64 * KPB + lane * KPB;
          if constexpr (KPB == 16) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
            for (int e = 0; e < 4; ++e) d.kw[tt][4 * hp + e] = w[e];
          } else {
            d.kw[tt][hp] = *reinterpret_cast<const uint32_t*>(src);
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < VNP; ++k) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(sb + LL::kStK + k * 1024 + lane * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) d.vw[4 * k + e] = w[e];
    }
    const unsigned char* ss = sb + LL::kStK + LL::kStV;
    d.ks = *reinterpret_cast<const u32x4*>(ss + tb * 16);
    d.kz = *reinterpret_cast<const u32x4*>(ss + oKZ + tb * 16);
    d.vs = *reinterpret_cast<const u32x4*>(ss + oVS + vs_at);
    d.vz = *reinterpret_cast<const u32x4*>(ss + oVZ + vs_at);
  };

  // One step: one key group.  score_step takes the group up to the P' operands
  // in LDS; value_step applies them to the group's value codes.
  // `tiles`: the step's Q' / P' operand area
  auto score_step = [&](const GroupLoads& d, unsigned char* tiles) {
    if (qtask) {
      u32x4 hi, lo;
      split8(qsv, d.ks, hi, lo);
      u32x4* qb = reinterpret_cast<u32x4*>(tiles);
      qb[qb_at(qb_entry)] = hi;
      qb[qb_at(qb_entry + 4)] = lo;
    }
    const float bias = zero_term(d.kz) * coefB;
    wave_lds_order();
    float v[8], pv[8];
    f32x4 sacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 bq = *reinterpret_cast<const u32x4*>(tiles + kk * 512 + qb_rd);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) sacc[tt] = mfma16(key_field<KB>(d.kw[tt], kk), bq, sacc[tt]);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * tt + r] = sacc[tt][r];
    }
    softmax_step(v, coefD, bias, pv, rescale_groups);

    // P' = p s (hi, lo) for the lane's (query, channel group, octet) and the
    // zero-point sum of the same task
    u32x4 hi, lo;
    split8(pv, d.vs, hi, lo);
    *reinterpret_cast<u32x4*>(tiles + LL::kPAOff + pa_hi) = hi;
    *reinterpret_cast<u32x4*>(tiles + LL::kPAOff + pa_lo) = lo;
    float zs = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const half2_t zz = as_half2(d.vz[k >> 1]);
      zs = fmaf(pv[k], float(zz[k & 1]), zs);
    }
    zacc += zs;
  };
  auto value_step = [&](const uint32_t (&vws)[VLW], const unsigned char* tiles) {
    wave_lds_order();
#pragma unroll
    for (int gc = 0; gc < NGV; ++gc) {
      const u32x4 ap = *reinterpret_cast<const u32x4*>(tiles + LL::kPAOff + pa_pos(gc, gq * 8 + (n & 7)) * 16);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int t = 2 * gc + half;
        const int chunk = t / TPW, sh = value_tile_shift<VB>(t % TPW);
        const bool down = (t % TPW) * VB != sh;
        u32x4 bv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t w = vws[m * NCH + chunk];
          bv[m] = (down ? w >> 8 : w) & (kVMask << sh);
        }
        oacc[t] = mfma16(ap, bv, oacc[t]);
      }
    }
    wave_lds_order();
  };

  {
    // Step i takes key group i from ring position i % D.  The prologue filled
    // positions 0 .. D - 1.  With D > 2 the copies of group i - 1 + D go to the
    // position step i - 1 was read from, before the wait for group i: those reads
    // have been consumed, so no wait on LDS is needed, and groups i + 1 ..
    // i + D - 1 stay in flight while the wave waits for group i.  With D == 2 step i's
    // own position takes the copies of group i + 2 right after it has been read
    // (after a wait for the reads).  Past the end of a short run the prologue's
    // copies came from an empty buffer.  The last step waits for all copies, so
    // the ring is idle afterwards.
    // Issue priority falls by one level per quarter of the unit's steps: the
    // waves of a SIMD are otherwise served oldest first and would finish far
    // apart; this way a wave that is ahead yields to the ones behind it.
    const int ns = nj;
    __builtin_amdgcn_s_setprio(3);
    const int q1 = ns / 4, q2 = ns / 2, q3 = (3 * ns) / 4;
    // step i at ring position pos_c == i % D: a compile-time constant where the
    // loop below is unrolled by D (every LDS address of a step is then a fixed
    // offset), a plain int otherwise
    auto one_step = [&](int i, auto pos_c) {
      const int pos = pos_c;
      if (i == q1) __builtin_amdgcn_s_setprio(2);
      if (i == q2) __builtin_amdgcn_s_setprio(1);
      if (i == q3) __builtin_amdgcn_s_setprio(0);
      if constexpr (D > 2) {
        // the position step i - 1 computed from is free (its reads were consumed
        // there): it takes group i - 1 + D before the wait, so D - 1 later groups
        // are in flight while the wave waits for group i
        const int prev = (pos + D - 1) % D;
        if (i >= 1 && i - 1 + D < ns) {
          wave_lds_order();
          stage_group(g0 + TS * (i - 1 + D), prev, true);
        }
      }
      // copy steps issued after group i: D - 1 (fewer near the end of the run;
      // waiting for more than needed there is harmless)
      wait_steps_ahead<kDmas, D - 1>(min(D - 1, ns - 1 - i));
      GroupLoads d;
      read_group(pos, d);
      if constexpr (D == 2) {
        wave_lds_sync();
        if (i + D < ns) stage_group(g0 + TS * (i + D), pos, true);
      }
      // the Q' / P' tiles overwrite the slot just read: LDS keeps the wave's
      // order, the compiler must keep it too
      wave_lds_order();
      unsigned char* tiles = LL::kInSlot ? stage + pos * LL::kSlot : smem + LL::oTiles;
      uint32_t vws[VLW];
#pragma unroll
      for (int k = 0; k < VLW; ++k) vws[k] = d.vw[k];
      score_step(d, tiles);
      value_step(vws, tiles);
    };
    static_assert(D == 2 || D == 3, "ring depth");
    if constexpr (lds_waves_per_simd<DK, DV, KB, VB, D>() <= 2) {
      for (int i0 = 0; i0 < ns; i0 += D) {
        one_step(i0, std::integral_constant<int, 0>{});
        if (i0 + 1 < ns) one_step(i0 + 1, std::integral_constant<int, 1>{});
        if constexpr (D > 2) {
          if (i0 + 2 < ns) one_step(i0 + 2, std::integral_constant<int, 2 % D>{});
        }
      }
    } else {
      // instances whose LDS admits 3 or 4 waves per SIMD (at most 168 or 128
      // registers): unrolled, the 128-register ones spill and the 168-register
      // ones measured no faster, so the position stays a variable.  It is hidden
      // from the compiler, which would otherwise keep one address per LDS access
      // advanced by a slot every step and corrected at the wrap (two vector
      // additions per access instead of one).
      for (int i = 0; i < ns; ++i) {
        int pos = i % D;
        asm volatile("" : "+s"(pos));
        one_step(i, pos);
      }
    }
    // a unit without key groups still issued (empty) copies into the ring
    wait_vmcnt<0>();
  }

  // --------------------------------------------------- retained fp16 rows
  // After the key groups (the order of tokens does not matter): the ring is idle
  // (the last group waited for every copy) and holds the probabilities PT; the
  // Q' tile takes the q hi/lo operand B2 again.
  if (unit < nRT) {
    // B2: q 2^-E split hi/lo, entry (kk*4 + gq)*8 + i + 4*part, channels of block
    // gq*KK + kk in natural order (dword d = channels 2d, 2d+1); query i = e % 4
    // is this lane's query.  The channels are the Q' task of lane 16 kk + 4 i + gq,
    // whose q 2^-E (qzv, after any rotation) is read across lanes.
    // (every lane runs the same passes, so that the cross-lane reads see all lanes;
    // lanes past the last entry read a lane in range and store nothing)
    for (int e0 = 0; e0 < KK * 32; e0 += 64) {
      const int e = e0 + lane;
      const int gqe = (e >> 3) & 3, kke = e >> 5, part = (e >> 2) & 1;
      const int src = (16 * kke + 4 * (e & 3) + gqe) & 63;
      float x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = __shfl(qzv[k], src);
      u32x4 v;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float x0 = x[2 * d], x1 = x[2 * d + 1];
        const half2_t hh = __builtin_convertvector(float2_t{x0, x1}, half2_t);
        const half2_t ll = __builtin_convertvector(float2_t{x0 - float(hh[0]), x1 - float(hh[1])}, half2_t);
        v[d] = __builtin_bit_cast(uint32_t, part ? ll : hh);
      }
      if (e < KK * 32) B2[e] = v;
    }
    wave_lds_sync();
    const uint8_t* kr = static_cast<const uint8_t*>(a.cache.k_fp16) + slab * a.r_stride * (DK * 2);
    const uint8_t* vr = static_cast<const uint8_t*>(a.cache.v_fp16) + slab * a.r_stride * (DV * 2);
    for (int rt = unit; rt < nRT; rt += U) {
      const int rbase = rt * 32;
      // the tile's value rows, loaded first so that their latency passes under the
      // scores and the softmax (channels 2 lane, 2 lane + 1 of each row)
      uint32_t vv[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int row = min(rbase + u, R - 1);
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vr + (uint32_t(row) * (DV * 2) + 4 * lane)));
      }
      f32x4 sacc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = min(rbase + 8 * (n >> 2) + 4 * tt + (n & 3), R - 1);
        sacc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 ak = *reinterpret_cast<const u32x4*>(kr + (uint32_t(row) * (DK * 2) + 16 * (gq * KK + kk)));
          sacc[tt] = mfma16(ak, B2[(kk * 4 + gq) * 8 + 4 * (rep & 1) + iq], sacc[tt]);
        }
      }
      // lane (n, gq): tile tt, register r -> token 8 gq + 4 tt + r
      float v[8], pv[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[4 * tt + r] = rbase + 8 * gq + 4 * tt + r < R ? sacc[tt][r] : -INFINITY;
      }
      softmax_step(v, coefB, 0.0f, pv, rescale_groups);
      if (rep == 0) {
        *reinterpret_cast<f32x4*>(PT + iq * 32 + 8 * gq) = f32x4{pv[0], pv[1], pv[2], pv[3]};
        *reinterpret_cast<f32x4*>(PT + iq * 32 + 8 * gq + 4) = f32x4{pv[4], pv[5], pv[6], pv[7]};
      }
      wave_lds_sync();
      // values on the VALU: lane owns channels 2 lane, 2 lane + 1 of every row
#pragma unroll
      for (int t0 = 0; t0 < 32; t0 += 8) {
#pragma unroll
        for (int u4 = 0; u4 < 8; u4 += 4) {
          f32x4 pq[kG];
#pragma unroll
          for (int i = 0; i < kG; ++i) pq[i] = *reinterpret_cast<const f32x4*>(PT + i * 32 + t0 + u4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const half2_t hv = as_half2(vv[t0 + u4 + u]);
#pragma unroll
            for (int i = 0; i < kG; ++i) {
              o_r[i][0] = fmaf(pq[i][u], float(hv[0]), o_r[i][0]);
              o_r[i][1] = fmaf(pq[i][u], float(hv[1]), o_r[i][1]);
            }
          }
        }
      }
      wave_lds_sync();
    }
  }

  // ------------------------------------------------------- the unit's result
  // The ring is idle now.  It takes the matrix-core output OM [4][DV] and the value
  // zero-point sums zsm [4][NGV]; the retained rows' part o_r stays in registers
  // (lane l owns channels 2l, 2l + 1 of every query, as in the output row).
  float* OM = reinterpret_cast<float*>(stage);
  float* zsm = OM + kG * DV;
  {
    // zero-point sums per (query, channel group): lanes 16 gq + 4 i + gc
    const float z16 = zacc + __shfl_xor(zacc, 16, 64);
    const float z = z16 + __shfl_xor(z16, 32, 64);
    if (gq == 0) zsm[iq * NGV + gcP] = z;
  }
  // Matrix-core accumulators: lane groups 0 and 1 hold the hi and lo rows of the 4
  // queries for column n of each tile.  One row swap of a pair of tiles (t, t + 1)
  // leaves hi + lo of tile t in lanes 0..15 and of tile t + 1 in lanes 16..31,
  // each written by exactly one lane (no atomics).
  static_assert(NV % 2 == 0, "tile pairs");
#pragma unroll
  for (int t = 0; t < NV; t += 2) {
    const float sc0 = 16777216.0f / float(1 << value_tile_shift<VB>(t % TPW));
    const float sc1 = 16777216.0f / float(1 << value_tile_shift<VB>((t + 1) % TPW));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto h2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(oacc[t][r] * sc0),
                                                       __float_as_uint(oacc[t + 1][r] * sc1), false, false);
      const float v = __uint_as_float(h2[0]) + __uint_as_float(h2[1]);
      if (gq < 2) OM[r * DV + 16 * (t + gq) + n] = v;
    }
  }
  wave_lds_sync();
  // l per query: the quads 16 gq + 4 i hold its tokens, two per lane: a sum over
  // each quad, then over the four octets
  const float lquad = quad_allreduce<false>(l_run);
  float lq[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i)
    lq[i] = readlane_f32(lquad, 4 * i) + readlane_f32(lquad, 16 + 4 * i) + readlane_f32(lquad, 32 + 4 * i) +
            readlane_f32(lquad, 48 + 4 * i);
  const int64_t qh0 = int64_t(b) * a.L.Hq + int64_t(h) * kG;
  // this unit's state per query, m, l: after the zero-point sums
  float* ML = zsm + kG * NGV;
  static_assert(4 * (kG * DV + kG * NGV + 2 * kG) <= LL::kBytes, "team state");
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    float2 o;
    const float2 om = *reinterpret_cast<const float2*>(OM + i * DV + 2 * lane);
    o.x = o_r[i][0] + om.x + zsm[i * NGV + (2 * lane) / 32];
    o.y = o_r[i][1] + om.y + zsm[i * NGV + (2 * lane + 1) / 32];
    if (U == 1) {
      const float inv = 1.0f / lq[i];
      o.x *= inv;
      o.y *= inv;
      *reinterpret_cast<float2*>(a.out + (qh0 + i) * DV + 2 * lane) = o;
    } else if (TS == kWavesPerGroup) {
      // kept for the team: each lane overwrites the elements it alone read
      *reinterpret_cast<float2*>(OM + i * DV + 2 * lane) = o;
    } else {
      // partial row of (query, unit): m, l, two unused floats, o[DV]
      float* row = a.partials + ((qh0 + i) * U + unit) * (DV + 4);
      *reinterpret_cast<float2*>(row + 4 + 2 * lane) = o;
      if (lane == 0) *reinterpret_cast<float4*>(row) = make_float4(m_q[i], lq[i], 0.0f, 0.0f);
    }
  }
  if (U > 1 && TS == kWavesPerGroup) {
    // The four units of the team combine their states by the merge's rule, wave w
    // taking query w, and the team writes one partial row per query (or, when the
    // team is the slab's only one, the output): a quarter of the rows for the
    // merge to read.  Every wave of the workgroup is a unit of the team, so all
    // of them reach the barrier.
    static_assert(kG == kWavesPerGroup, "one query per wave");
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        ML[i] = m_q[i];
        ML[kG + i] = lq[i];
      }
    }
    __syncthreads();
    const int i = wave;
    float mw[kWavesPerGroup], lw[kWavesPerGroup];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      const float* mlw = reinterpret_cast<const float*>(lds_all + w * LL::kBytes) + kG * DV + kG * NGV;
      mw[w] = mlw[i];
      lw[w] = mlw[kG + i];
      M = fmaxf(M, mw[w]);
    }
    float2 o = make_float2(0.0f, 0.0f);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) {
      const float wt = lse_weight(mw[w], M);
      const float2 ow = *reinterpret_cast<const float2*>(reinterpret_cast<const float*>(lds_all + w * LL::kBytes) +
                                                         i * DV + 2 * lane);
      o.x = fmaf(wt, ow.x, o.x);
      o.y = fmaf(wt, ow.y, o.y);
      L = fmaf(wt, lw[w], L);
    }
    const int T = U / TS;
    if (T == 1) {
      const float inv = 1.0f / L;
      *reinterpret_cast<float2*>(a.out + (qh0 + i) * DV + 2 * lane) = make_float2(o.x * inv, o.y * inv);
    } else {
      // partial row of (query, team): m, l, two unused floats, o[DV]
      float* row = a.partials + ((qh0 + i) * T + team) * (DV + 4);
      *reinterpret_cast<float2*>(row + 4 + 2 * lane) = o;
      if (lane == 0) *reinterpret_cast<float4*>(row) = make_float4(M, L, 0.0f, 0.0f);
    }
  }
}

// Opt an instance into more than the default 64 KB of LDS (gfx950 has 160 KB per
// compute unit), once per device: the attribute stays set for the process.
template <int DK, int DV, int KB, int VB, int D>
hipError_t lds_optin(int dev, int bytes) {
  static std::atomic<uint64_t> done{0};
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_mfma_kernel<DK, DV, KB, VB, D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

template <int DK, int DV, int KB, int VB, int D>
hipError_t launch_depth(DecodeArgs a, hipStream_t stream, int dev, const DecodePlan& plan) {
  constexpr size_t lds = size_t(kWavesPerGroup) * Lds<DK, DV, KB, VB, D>::kBytes;
  static_assert(lds <= 160 * 1024, "LDS budget");
  a.units = plan.units;
  a.ranks = plan.ranks;
  {
    // the teams' run starts, as the kernel would compute them (team_start)
    const int U = a.units, TS = (U % kWavesPerGroup) == 0 ? kWavesPerGroup : 1, T = U / TS;
    const int nRT = (a.L.R + 31) / 32, tq = nRT / U, tm = nRT % U;
    const int tc16 = tile_cost16<DK, DV, KB, VB>(a.L);
    a.n_team_first = 0;
    if (T <= kMaxTeamTable) {
      for (int t = 0; t <= T; ++t) a.team_first[t] = team_start(t, T, TS, a.L.n_groups, a.ranks, tq, tm, tc16);
      a.n_team_first = T + 1;
    }
  }
  if constexpr (lds > 64 * 1024) {
    const hipError_t e = lds_optin<DK, DV, KB, VB, D>(dev, int(lds));
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (plan.waves + kWavesPerGroup - 1) / kWavesPerGroup;
  if (a.kernel_start || a.kernel_stop)
    return launch_decode_timed(reinterpret_cast<const void*>(&decode_mfma_kernel<DK, DV, KB, VB, D>),
                               dim3(unsigned(blocks)), dim3(64 * kWavesPerGroup), lds, stream, a);
  hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, KB, VB, D>), dim3(unsigned(blocks)), dim3(64 * kWavesPerGroup), lds,
                     stream, a);
  return hipGetLastError();
}

template <int DK, int DV, int KB, int VB>
hipError_t run_one(const DecodeArgs& a, hipStream_t stream, int dev, int cus, DecodePlan* plan, bool launch) {
  // Units are cut as far as the 2-deep ring's LDS keeps every wave resident (up to
  // 16 waves per compute unit).  With the non-temporal copies the 128K workload
  // runs faster as 4096 half-length runs on a 2-deep ring than as 2048 long ones on
  // a 3-deep ring (cold calls 103.6 -> 101.0 us p50, inside the step 103.9 -> 100.0,
  // interleaved); with plain copies it had been the other way round.  The ring has
  // 3 steps where the grid puts at most 2 waves on a SIMD and that LDS still lets
  // the whole grid be resident at once, else 2: with 4 waves per SIMD the other
  // waves keep enough copies in flight (32K workload, 4096 waves: 156.9 -> 153.9 us
  // p50 with the 2-deep ring as cold calls, 181.4 -> 178.1 back to back); with 2
  // per SIMD the third slot pays (4K workload 16.4 -> 16.0 us, 16K 47.2 -> 46.8).
  // With a grid of 2048 waves, 4 steps (more copies in flight) measured no faster
  // on the 128K workload and slower on the 16K and 4K ones (50.5 against 51.1 us,
  // 17.7 against 18.5), and a 5th no faster either.
  const int per_cu = 4 * lds_waves_per_simd<DK, DV, KB, VB, 2>();
  const int units = decode_mfma_units(a.L, a.P, int64_t(cus) * (per_cu < 16 ? per_cu : 16));
  const int64_t waves = int64_t(units) * a.L.B * a.L.Hkv;
  const int64_t simds = int64_t(cus) * 4;
  int depth = 2, per_simd = lds_waves_per_simd<DK, DV, KB, VB, 2>();
  if (waves <= simds * std::min(2, lds_waves_per_simd<DK, DV, KB, VB, 3>())) {
    depth = 3;
    per_simd = lds_waves_per_simd<DK, DV, KB, VB, 3>();
  }
  plan->kernel = KVQ_KERNEL_MFMA;
  plan->units = units;
  // teams of four units combine their states in the kernel (one partial row per team)
  plan->rows = units % kWavesPerGroup == 0 ? units / kWavesPerGroup : units;
  plan->depth = depth;
  plan->ranks = int(std::min<int64_t>(per_simd, std::max<int64_t>(1, (waves + simds - 1) / simds)));
  plan->waves = waves;
  if (!launch) return hipSuccess;
  if (depth == 3) return launch_depth<DK, DV, KB, VB, 3>(a, stream, dev, *plan);
  return launch_depth<DK, DV, KB, VB, 2>(a, stream, dev, *plan);
}

template <int DK, int DV>
hipError_t run_bits(const DecodeArgs& a, hipStream_t stream, int dev, int cus, DecodePlan* plan, bool launch) {
  const int kb = a.L.k_bits, vb = a.L.v_bits;
  // key rows must give every lane at least 4 bytes of a tile (staged as dwords)
#define KVQ_BITS_CASE(K_, V_)                                                          \
  if constexpr (DK * K_ / 32 >= 4) {                                                   \
    if (kb == K_ && vb == V_) return run_one<DK, DV, K_, V_>(a, stream, dev, cus, plan, launch); \
  }
  KVQ_BITS_CASE(2, 2) KVQ_BITS_CASE(2, 4) KVQ_BITS_CASE(2, 8)
  KVQ_BITS_CASE(4, 2) KVQ_BITS_CASE(4, 4) KVQ_BITS_CASE(4, 8)
  KVQ_BITS_CASE(8, 2) KVQ_BITS_CASE(8, 4) KVQ_BITS_CASE(8, 8)
#undef KVQ_BITS_CASE
  return hipErrorInvalidValue;  // unreachable for a shape mfma_takes accepts
}

}  // namespace

hipError_t device_cus(int* dev, int* cus) {
  static std::atomic<int> cached[64];
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return e;
  if (*dev >= 0 && *dev < 64) {
    const int c = cached[*dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, *dev);
  if (e != hipSuccess) return e;
  if (*cus < 1) return hipErrorInvalidDevice;
  if (*dev >= 0 && *dev < 64) cached[*dev].store(*cus, std::memory_order_relaxed);
  return hipSuccess;
}

bool mfma_takes(const kvq_layout& L, int P) {
  if (L.Hq != kG * L.Hkv || L.Dv != 128) return false;
  if (L.Dk != 32 && L.Dk != 64 && L.Dk != 128) return false;
  const auto ok_bits = [](int b) { return b == 2 || b == 4 || b == 8; };
  if (!ok_bits(L.k_bits) || !ok_bits(L.v_bits) || L.Dk * L.k_bits / 32 < 4) return false;
  // per-slab offsets are 32-bit in this kernel, and so is the wave index
  const int64_t widest = L.Dk > L.Dv ? L.Dk : L.Dv;
  if (int64_t(L.Tq) * widest >= (int64_t(1) << 31) || int64_t(L.R) * widest * 2 >= (int64_t(1) << 31)) return false;
  return int64_t(kMaxUnitsPerPartition) * P * L.B * L.Hkv < (int64_t(1) << 31);
}

hipError_t mfma_decode(const DecodeArgs& a, hipStream_t stream, DecodePlan* plan, bool launch) {
  int dev = 0, cus = 0;
  const hipError_t e = device_cus(&dev, &cus);
  if (e != hipSuccess) return e;
  switch (a.L.Dk) {
    case 32: return run_bits<32, 128>(a, stream, dev, cus, plan, launch);
    case 64: return run_bits<64, 128>(a, stream, dev, cus, plan, launch);
    case 128: return run_bits<128, 128>(a, stream, dev, cus, plan, launch);
    default: return hipErrorInvalidValue;  // unreachable for a shape mfma_takes accepts
  }
}

}  // namespace kvq
