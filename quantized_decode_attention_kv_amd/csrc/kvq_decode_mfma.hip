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
//   scores  s_t = sum_c (q_c s_c) n_tc + sum_c q_c z_c                (per key group)
//   values  o_c = sum_t (p_t s_t,g) n_tc + sum_t p_t z_t,g   (g = 32-channel group of c)
// The folded operands q_c s_c and p_t s_t,g are split into fp16 hi + lo parts
// (each rounded to nearest, about 22 significant bits together).
//
// One wave owns every fourth key group of the workgroup's partition and keeps one
// group's loads in flight while it computes the previous one.  Per group:
//   1. Q' = q s (hi, lo) for 64 (query, 8-channel block) tasks, one per lane, into
//      a wave-private LDS tile;
//   2. scores S^T[token, column] = codes (A: 16 tokens x 32 channels) x Q' (B), two
//      16-token tiles.  Column n holds query n%4, part (n/4)%2, so one DPP rotate
//      adds the lo part to the hi part and every lane ends up with the scores of
//      query n%4.  Tile rows are ordered so that lane group j holds tokens
//      8j..8j+7;
//   3. the key zero-point term sum_c q_c z_c comes from a 16-group batch MFMA
//      (A = the zero points of 16 groups, B = q split hi/lo) done once per 16
//      groups, read back from LDS;
//   4. online softmax in the log2 domain on the 8 scores of each lane; the running
//      maximum of a query only moves (and the state is rescaled) when a score
//      exceeds it by more than 2^kHeadroom, so most groups skip the rescale;
//   5. P' = p s (hi, lo) for 64 (query, channel group, 8-token octet) tasks, again
//      one per lane and already holding the probabilities they need, into LDS;
//   6. values O[(query, part), channel] += P' (A) x codes (B), eight 16-channel
//      tiles.  A lane's B operand for tile t is its code word of that tile's
//      chunk masked to the tile's bit slot: one AND per operand register (plus
//      one shift per word for the slots above the mantissa).
// Retained fp16 rows (recent window, log-spaced tokens) are folded into the same
// online state first: scores on the MFMA (A = fp16 key rows), values on the VALU.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_decode_common.hpp"
#include "kvq_internal.hpp"

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

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c, 0,
                                                0, 0);
}

// v plus the value of the lane four columns away inside its row of 16.  Columns
// n and n^4 hold the two parts of the same query and the pattern repeats every 8
// columns, so either rotation direction pairs them.
__device__ __forceinline__ float add_ror4(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
}
// Reinterpret a packed fp16 pair.  Takes its argument by value: clang's
// __builtin_bit_cast applied directly to an element of an ext_vector_type lvalue
// reads element 0 whatever the index.
__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// LDS bytes of the kernel: [shared head][4 wave areas], reused for the epilogue
template <int DK, int DV>
struct Lds {
  static constexpr int KK = DK / 32, NGV = DV / 32;
  static constexpr int kQs = kG * DK * 4;      // scaled q, fp32 [4][DK]
  static constexpr int kQexp = 16;             // [4] power-of-two query scalings
  static constexpr int kB2 = KK * 32 * 16;     // q hi/lo operand tile
  static constexpr int kShared = kQs + kQexp + kB2;
  static constexpr int kQB = KK * 32 * 16;     // Q' operand tile
  static constexpr int kPA = NGV * 32 * 16;    // P' operand tile
  static constexpr int kBT = kG * 16 * 4;      // zero-point terms of 16 groups
  static constexpr int kPT = kG * 32 * 4;      // retained-row probabilities
  static constexpr int kWave = kQB + kPA + kBT + kPT;
  static constexpr int kLoop = kShared + kDecodeWaves * kWave;
  // epilogue: wave states [4][4][DV + 2], zero sums [4][4][NGV], res [4][DV + 2]
  static constexpr int kSt = kDecodeWaves * kG * (DV + 2) * 4;
  static constexpr int kZs = kDecodeWaves * kG * NGV * 4;
  static constexpr int kRes = kG * (DV + 2) * 4;
  static constexpr int kMerge = kShared + kSt + kZs + kRes;
  static constexpr int kBytes = kLoop > kMerge ? kLoop : kMerge;
};

template <int DK, int DV, int KB, int VB>
__global__ __launch_bounds__(kDecodeThreads) void decode_mfma_kernel(const DecodeArgs a) {
  using LL = Lds<DK, DV>;
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
  static_assert(DV == 128 && NV % TPW == 0 && KLB >= 2 && DK % 32 == 0 && DK <= 256, "shape");

  extern __shared__ __align__(16) unsigned char smem[];
  float* qs_lds = reinterpret_cast<float*>(smem);                            // [4][DK]
  float* qexp = reinterpret_cast<float*>(smem + LL::kQs);                    // [4]
  u32x4* B2 = reinterpret_cast<u32x4*>(smem + LL::kQs + LL::kQexp);          // [KK*4][8]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, gq = lane >> 4;
  unsigned char* wb = smem + LL::kShared + wave * LL::kWave;
  u32x4* QB = reinterpret_cast<u32x4*>(wb);                                  // [KK*4][8]
  u32x4* PA = reinterpret_cast<u32x4*>(wb + LL::kQB);                        // [NGV*4][8]
  float* BT = reinterpret_cast<float*>(wb + LL::kQB + LL::kPA);              // [4][16]
  float* PT = reinterpret_cast<float*>(wb + LL::kQB + LL::kPA + LL::kBT);    // [4][32]

  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nG = a.L.n_groups, R = a.L.R, P = a.P;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  const int g0 = int(int64_t(p) * nG / P), g1 = int(int64_t(p + 1) * nG / P);
  const int nRT = (R + 31) / 32;  // 32-row tiles of retained rows
  const int rt0 = int(int64_t(p) * nRT / P), rt1 = int(int64_t(p + 1) * nRT / P);

  // ---------------------------------------------------------------- set-up
  for (int idx = tid; idx < kG * DK; idx += kDecodeThreads)
    qs_lds[idx] = a.scale * kLog2e * load_q_any(a.q, a.q_dtype, (int64_t(b) * a.L.Hq + int64_t(h) * kG) * DK + idx);
  __syncthreads();
  if (wave == 0) {
    // per query: 2^-E with E >= 0 the smallest exponent such that |q * 2^-E| <= 1,
    // keeping q_c s_c inside the fp16 range
    for (int i = 0; i < kG; ++i) {
      float mx = 0.0f;
      for (int c = lane; c < DK; c += 64) mx = fmaxf(mx, fabsf(qs_lds[i * DK + c]));
      mx = wave_max(mx);
      if (lane == 0) {
        int e = 0;
        frexpf(mx, &e);
        qexp[i] = mx > 1.0f ? ldexpf(1.0f, -e) : 1.0f;
      }
    }
  }
  __syncthreads();
  // B2: q 2^-E split hi/lo, entry (kk*4 + gq)*8 + i + 4*part, channels of block
  // gq*KK + kk in natural order (dword d = channels 2d, 2d+1)
  for (int e = tid; e < KK * 32; e += kDecodeThreads) {
    const int c8 = e & 7, gqe = (e >> 3) & 3, kke = e >> 5;
    const int i = c8 & 3, part = c8 >> 2;
    const float* src = qs_lds + i * DK + 8 * (gqe * KK + kke);
    u32x4 v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float x0 = src[2 * d] * qexp[i], x1 = src[2 * d + 1] * qexp[i];
      const half2_t hh = __builtin_convertvector(float2_t{x0, x1}, half2_t);
      const half2_t ll = __builtin_convertvector(float2_t{x0 - float(hh[0]), x1 - float(hh[1])}, half2_t);
      v[d] = __builtin_bit_cast(uint32_t, part ? ll : hh);
    }
    B2[e] = v;
  }

  // Q' task of this lane: (block kk_t of lane group gq_t, query i_t); q 2^-E
  // divided by the code scale of each operand slot
  const int kk_t = lane >> 4, gq_t = (lane >> 2) & 3, i_t = lane & 3;
  const bool qtask = kk_t < KK;
  const int tb = gq_t * KK + (qtask ? kk_t : 0);
  float qsv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    qsv[k] = qtask ? qs_lds[i_t * DK + 8 * tb + k] * qexp[i_t] * (1.0f / key_code_scale<KB>(k & 3)) : 0.0f;
  const int qb_entry = ((qtask ? kk_t : 0) * 4 + gq_t) * 8 + i_t;
  // score columns: query iq = n % 4
  const int iq = n & 3;
  const float coefD = 16777216.0f / qexp[iq];  // codes are n 2^-24; q was scaled by 2^-E
  const float coefB = 1.0f / qexp[iq];
  // P' task: (query iq, channel group n / 4, octet gq)
  const int gcP = n >> 2;
  const int pa_entry = (gcP * 4 + gq) * 8 + iq;
  __syncthreads();  // B2 complete

  // online-softmax state: reference maxima per query (wave-uniform) and this
  // lane's copy for its query; l over the lane's tokens; value accumulators
  float m_q[kG];
#pragma unroll
  for (int i = 0; i < kG; ++i) m_q[i] = -INFINITY;
  float m_lane = -INFINITY, l_run = 0.0f, zacc = 0.0f;
  f32x4 oacc[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t) oacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float o_r[kG][2];  // retained rows: channels 2 lane, 2 lane + 1
#pragma unroll
  for (int i = 0; i < kG; ++i) o_r[i][0] = o_r[i][1] = 0.0f;

  // Softmax update of 8 new scores per lane: v = raw combined MFMA outputs,
  // score = v * coef + bias (log2 domain).  Returns the probabilities relative to
  // the (possibly moved) reference maximum.
  auto softmax_step = [&](const float (&v)[8], float coef, float bias, float (&pv)[8]) {
    const float bterm = bias - m_lane;
    float sv[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sv[k] = fmaf(v[k], coef, bterm);
      mloc = fmaxf(mloc, sv[k]);
    }
    if (__builtin_expect(__any(mloc > float(kHeadroom)), 0)) {
      // some score left the headroom: move those references to the group maxima
      // (queries repeat every 4 columns; the 4 lane groups hold different tokens)
      float sabs[8];
      float mab = -INFINITY;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        sabs[k] = fmaf(v[k], coef, bias);
        mab = fmaxf(mab, sabs[k]);
      }
      float alpha[kG];
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        float mg = readlane_f32(mab, i);
#pragma unroll
        for (int j = 1; j < 4; ++j) mg = fmaxf(mg, readlane_f32(mab, 16 * j + i));
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
#pragma unroll
      for (int t = 0; t < NV; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[t][r] *= alpha[r];
      }
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        o_r[i][0] *= alpha[i];
        o_r[i][1] *= alpha[i];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) sv[k] = sabs[k] - m_lane;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pv[k] = fast_exp2(sv[k]);
      l_run += pv[k];
    }
  };

  // ----------------------------------------------- retained fp16 rows first
  {
    const uint8_t* kr = static_cast<const uint8_t*>(a.cache.k_fp16) + slab * int64_t(R) * (DK * 2);
    const uint8_t* vr = static_cast<const uint8_t*>(a.cache.v_fp16) + slab * int64_t(R) * (DV * 2);
    for (int rt = rt0 + wave; rt < rt1; rt += kDecodeWaves) {
      const int rbase = rt * 32;
      f32x4 sacc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = min(rbase + 8 * (n >> 2) + 4 * tt + (n & 3), R - 1);
        sacc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 ak = *reinterpret_cast<const u32x4*>(kr + (uint32_t(row) * (DK * 2) + 16 * (gq * KK + kk)));
          sacc[tt] = mfma16(ak, B2[(kk * 4 + gq) * 8 + (n & 7)], sacc[tt]);
        }
      }
      // lane (n, gq): tile tt, register r -> token 8 gq + 4 tt + r
      float v[8], pv[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = add_ror4(sacc[tt][r]);
          v[4 * tt + r] = rbase + 8 * gq + 4 * tt + r < R ? x : -INFINITY;
        }
      }
      softmax_step(v, coefB, 0.0f, pv);
      if (n < kG) {
        *reinterpret_cast<f32x4*>(PT + n * 32 + 8 * gq) = f32x4{pv[0], pv[1], pv[2], pv[3]};
        *reinterpret_cast<f32x4*>(PT + n * 32 + 8 * gq + 4) = f32x4{pv[4], pv[5], pv[6], pv[7]};
      }
      wave_lds_sync();
      // values on the VALU: lane owns channels 2 lane, 2 lane + 1 of every row
#pragma unroll
      for (int t0 = 0; t0 < 32; t0 += 8) {
        uint32_t vv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = min(rbase + t0 + u, R - 1);
          vv[u] = *reinterpret_cast<const uint32_t*>(vr + (uint32_t(row) * (DV * 2) + 4 * lane));
        }
#pragma unroll
        for (int u4 = 0; u4 < 8; u4 += 4) {
          f32x4 pq[kG];
#pragma unroll
          for (int i = 0; i < kG; ++i) pq[i] = *reinterpret_cast<const f32x4*>(PT + i * 32 + t0 + u4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const half2_t hv = as_half2(vv[u4 + u]);
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

  // ------------------------------------------------------------ key groups
  // per-slab bases (wave-uniform) and 32-bit lane offsets
  const uint8_t* kbase = static_cast<const uint8_t*>(a.cache.k_codes) + slab * int64_t(a.L.Tq) * KROW;
  const uint16_t* ksbase = static_cast<const uint16_t*>(a.cache.k_scale) + slab * int64_t(nG) * DK;
  const uint16_t* kzbase = static_cast<const uint16_t*>(a.cache.k_zero) + slab * int64_t(nG) * DK;
  const uint32_t* vbase = static_cast<const uint32_t*>(a.cache.v_codes) + slab * int64_t(nG) * (DV * VB);
  const uint16_t* vsbase = static_cast<const uint16_t*>(a.cache.v_scale) + slab * int64_t(nG) * DV;
  const uint16_t* vzbase = static_cast<const uint16_t*>(a.cache.v_zero) + slab * int64_t(nG) * DV;
  uint32_t koff[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) koff[tt] = uint32_t(8 * (n >> 2) + 4 * tt + (n & 3)) * KROW + gq * KLB;
  const uint32_t voff = uint32_t(lane) * VLW;
  const uint32_t ksoff = uint32_t(8 * tb);
  const uint32_t vsoff = uint32_t(gcP * 32 + 8 * gq);

  // everything one key group needs from HBM, held in registers so the next
  // group's loads are in flight while the current one is computed
  struct GroupLoads {
    uint32_t kw[2][KLW];  // key codes of tiles 0, 1 (row n = token 8(n/4) + 4tt + n%4)
    uint32_t vw[VLW];     // value code words: pair m, chunk c at m*NCH + c
    u32x4 ks;             // key scales of the lane's Q' block
    u32x4 vs, vz;         // value scale / zero of the lane's P' channel group, tokens 8gq..
  };
  // Branch-free: every lane issues the same loads, so the compiler can count
  // outstanding loads and wait only for the current group's.
  auto load_group = [&](int g, GroupLoads& d) {
    const uint8_t* kg = kbase + uint32_t(g) * (32 * KROW);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) load_bytes<KLB>(kg + koff[tt], d.kw[tt]);
    const uint32_t* vg = vbase + uint32_t(g) * (DV * VB);
#pragma unroll
    for (int k = 0; k < VLW / 4; ++k) {
      const u32x4 w4 = *reinterpret_cast<const u32x4*>(vg + voff + 4 * k);
      d.vw[4 * k] = w4[0];
      d.vw[4 * k + 1] = w4[1];
      d.vw[4 * k + 2] = w4[2];
      d.vw[4 * k + 3] = w4[3];
    }
    d.ks = *reinterpret_cast<const u32x4*>(ksbase + uint32_t(g) * DK + ksoff);
    d.vs = *reinterpret_cast<const u32x4*>(vsbase + uint32_t(g) * DV + vsoff);
    d.vz = *reinterpret_cast<const u32x4*>(vzbase + uint32_t(g) * DV + vsoff);
  };

  const int nj = g1 - g0 - wave > 0 ? (g1 - g0 - wave + kDecodeWaves - 1) / kDecodeWaves : 0;
  auto group_of = [&](int j) { return g0 + wave + kDecodeWaves * j; };

  // zero-point terms of the wave's groups j0 .. j0 + 15: A = the zero points of
  // the 16 groups (row = group), B = q split hi/lo; into BT [query][group]
  auto bias_batch = [&](int j0) {
    const int gr = group_of(min(j0 + n, nj - 1));
    const uint16_t* zr = kzbase + uint32_t(gr) * DK;
    f32x4 db = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 az = *reinterpret_cast<const u32x4*>(zr + 8 * (gq * KK + kk));
      db = mfma16(az, B2[(kk * 4 + gq) * 8 + (n & 7)], db);
    }
    f32x4 bz;
#pragma unroll
    for (int r = 0; r < 4; ++r) bz[r] = add_ror4(db[r]) * coefB;
    if (n < kG) *reinterpret_cast<f32x4*>(BT + n * 16 + 4 * gq) = bz;
  };

  auto process_group = [&](const GroupLoads& d, int j) {
    if (qtask) {
      u32x4 hi, lo;
      split8(qsv, d.ks, hi, lo);
      QB[qb_entry] = hi;
      QB[qb_entry + 4] = lo;
    }
    wave_lds_sync();
    const float bias = BT[iq * 16 + (j & 15)];
    f32x4 sacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 bq = QB[(kk * 4 + gq) * 8 + (n & 7)];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) sacc[tt] = mfma16(key_field<KB>(d.kw[tt], kk), bq, sacc[tt]);
    }
    float v[8], pv[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * tt + r] = add_ror4(sacc[tt][r]);
    }
    softmax_step(v, coefD, bias, pv);

    // P' = p s (hi, lo) for the lane's (query, channel group, octet) and the
    // zero-point sum of the same task
    {
      u32x4 hi, lo;
      split8(pv, d.vs, hi, lo);
      PA[pa_entry] = hi;
      PA[pa_entry + 4] = lo;
      float zs = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const half2_t zz = as_half2(d.vz[k >> 1]);
        zs = fmaf(pv[k], float(zz[k & 1]), zs);
      }
      zacc += zs;
    }
    wave_lds_sync();
#pragma unroll
    for (int gc = 0; gc < NGV; ++gc) {
      const u32x4 ap = PA[(gc * 4 + gq) * 8 + (n & 7)];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int t = 2 * gc + half;
        const int chunk = t / TPW, sh = value_tile_shift<VB>(t % TPW);
        const bool down = (t % TPW) * VB != sh;
        u32x4 bv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t w = d.vw[m * NCH + chunk];
          bv[m] = (down ? w >> 8 : w) & (kVMask << sh);
        }
        oacc[t] = mfma16(ap, bv, oacc[t]);
      }
    }
  };

  {
    // the prefetch past the last group re-reads the last group (always in bounds)
    GroupLoads buf0, buf1;
    if (nj > 0) load_group(group_of(0), buf0);
    for (int j = 0; j < nj; j += 2) {
      if ((j & 15) == 0) bias_batch(j);
      load_group(group_of(min(j + 1, nj - 1)), buf1);
      process_group(buf0, j);
      if (j + 1 >= nj) break;
      load_group(group_of(min(j + 2, nj - 1)), buf0);
      process_group(buf1, j + 1);
    }
  }

  // -------------------------------------------- combine the 4 wave states
  __syncthreads();  // every wave is out of its loops; the loop LDS is free now
  float* st = reinterpret_cast<float*>(smem + LL::kShared);                       // [4][4][DV + 2]
  float* zsm = reinterpret_cast<float*>(smem + LL::kShared + LL::kSt);            // [4][4][NGV]
  float* res = reinterpret_cast<float*>(smem + LL::kShared + LL::kSt + LL::kZs);  // [4][DV + 2]
  {
    float* sw = st + wave * kG * (DV + 2);
    // l per query: lanes i, 16 + i, 32 + i, 48 + i hold its four token octets
    float lq[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i)
      lq[i] = readlane_f32(l_run, i) + readlane_f32(l_run, 16 + i) + readlane_f32(l_run, 32 + i) +
              readlane_f32(l_run, 48 + i);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < kG; ++i) {
        sw[i * (DV + 2)] = m_q[i];
        sw[i * (DV + 2) + 1] = lq[i];
      }
    }
    // zero-point sums per (query, channel group): lanes 16 gq + 4 gc + i
    const float z16 = zacc + __shfl_xor(zacc, 16, 64);
    const float z = z16 + __shfl_xor(z16, 32, 64);
    if (gq == 0) zsm[(wave * kG + iq) * NGV + gcP] = z;
    // matrix-core output: lane (n, 0) holds the hi rows, lane (n, 1) the lo rows
    // of column n; tile t's codes carried 2^(slot * VB)
    if (gq == 0) {
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const float sc = 16777216.0f / float(1 << value_tile_shift<VB>(t % TPW));
#pragma unroll
        for (int r = 0; r < 4; ++r) sw[r * (DV + 2) + 2 + 16 * t + n] = oacc[t][r] * sc;
      }
    }
    wave_lds_sync();
    if (gq == 1) {
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        const float sc = 16777216.0f / float(1 << value_tile_shift<VB>(t % TPW));
#pragma unroll
        for (int r = 0; r < 4; ++r) sw[r * (DV + 2) + 2 + 16 * t + n] += oacc[t][r] * sc;
      }
    }
    wave_lds_sync();
    // zero-point terms and the retained rows' values
#pragma unroll
    for (int i = 0; i < kG; ++i) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * lane + e;
        sw[i * (DV + 2) + 2 + c] += zsm[(wave * kG + i) * NGV + c / 32] + o_r[i][e];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kG * DV; idx += kDecodeThreads) {
    const int i = idx / DV, c = idx - i * DV;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, st[(w * kG + i) * (DV + 2)]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float* e = st + (w * kG + i) * (DV + 2);
      const float wt = lse_weight(e[0], M);
      L += wt * e[1];
      O += wt * e[2 + c];
    }
    res[i * (DV + 2) + 2 + c] = O;
    if (c == 0) {
      res[i * (DV + 2)] = M;
      res[i * (DV + 2) + 1] = L;
    }
  }
  __syncthreads();
  finish_partition(a, kG, b, h, p, res);
}

template <int DK, int DV, int KB, int VB>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  constexpr size_t lds = Lds<DK, DV>::kBytes;
  static_assert(lds <= 64 * 1024, "LDS budget");
  const dim3 grid(unsigned(a.P), unsigned(a.L.Hkv), unsigned(a.L.B));
  hipLaunchKernelGGL((decode_mfma_kernel<DK, DV, KB, VB>), grid, dim3(kDecodeThreads), lds, stream, a);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bits(const DecodeArgs& a, hipStream_t stream) {
  const int kb = a.L.k_bits, vb = a.L.v_bits;
#define KVQ_BITS_CASE(K_, V_) \
  if (kb == K_ && vb == V_) return launch_one<DK, DV, K_, V_>(a, stream);
  KVQ_BITS_CASE(2, 2) KVQ_BITS_CASE(2, 4) KVQ_BITS_CASE(2, 8)
  KVQ_BITS_CASE(4, 2) KVQ_BITS_CASE(4, 4) KVQ_BITS_CASE(4, 8)
  KVQ_BITS_CASE(8, 2) KVQ_BITS_CASE(8, 4) KVQ_BITS_CASE(8, 8)
#undef KVQ_BITS_CASE
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (a.L.Hq != kG * a.L.Hkv || a.L.Dv != 128) return hipErrorNotSupported;
  // per-slab offsets are 32-bit in this kernel
  const int64_t widest = a.L.Dk > a.L.Dv ? a.L.Dk : a.L.Dv;
  if (int64_t(a.L.Tq) * widest >= (int64_t(1) << 31) || int64_t(a.L.R) * widest * 2 >= (int64_t(1) << 31))
    return hipErrorNotSupported;
  switch (a.L.Dk) {
    case 32: return launch_bits<32, 128>(a, stream);
    case 64: return launch_bits<64, 128>(a, stream);
    case 128: return launch_bits<128, 128>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace kvq
