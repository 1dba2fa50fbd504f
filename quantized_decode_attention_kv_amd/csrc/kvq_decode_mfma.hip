// kv_decode_attn, matrix-core kernel for gfx950.
//
// Same computation as the generic kernel (single-token decode attention read
// straight from the packed cache; see kvq_decode_generic.hip), restructured so the
// two dot products run on v_mfma_f32_16x16x32_f16 and the vector ALUs only unpack
// codes and scale small operand tiles.
//
// Codes enter the MFMA unconverted: a b-bit code n (b <= 8) placed in the low bits
// of an fp16 lane is the subnormal n * 2^-24, exactly.  Products with fp16
// operands are exact and accumulate in fp32, so every result is scaled by 2^24 at
// the end.  Per-channel key scales and per-token value scales are folded into the
// other operand, and the zero points become one bias per row:
//   scores  s_t = sum_c (q_c s_c) n_tc + sum_c q_c z_c                 (per key group)
//   values  o_c = sum_t (p_t s_t,g) n_tc + sum_t p_t z_t,g   (g = channel group of c)
// The folded operands q_c s_c and p_t s_t,g are split into fp16 hi + lo parts
// (about 21 significant bits together) occupying two MFMA columns (scores) or rows
// (values) each, so the G query heads of a KV head use 2G of the 16 columns.
//
// One wave processes one 32-token key group at a time:
//   1. scores: S^T[token, (query, part)] = codes (A, 16 tokens x 32 channels per
//      step) x Q' (B); two 16-token tiles, Dk/32 steps each.  Tile rows are
//      ordered so that lane group j (lanes 16j..16j+15) ends up holding tokens
//      8j..8j+7 of the group;
//   2. online softmax in the log2 domain on those 8 scores per lane;
//   3. values: O[(query, part), channel] += P' (A, rows = (query, part), K = the
//      32 tokens) x codes (B, 16 channels of one channel group per tile).  Lane
//      group j supplies tokens 8j..8j+7, which is why value codes are stored per
//      8-token octet and channel: a lane's operand is one contiguous field.
// Q' and P' are computed once per group by the lanes that own them and handed to
// the operand layout through LDS (wave-private, no barriers).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_decode_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Order LDS traffic of one wave: the wave's own LDS accesses complete in issue
// order, so a compiler barrier plus a wait for outstanding LDS operations suffices.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ half8 as_half8(u32x4 v) { return __builtin_bit_cast(half8, v); }

// 8 codes -> 4 dwords, dword m = (code m, code m+4) as fp16 subnormals.
// 2-bit: the 16-bit field sits in half `hi` of w.
__device__ __forceinline__ u32x4 unpack2(uint32_t w, int hi) {
  const uint32_t y = __builtin_amdgcn_perm(w, w, hi ? 0x0C030C02u : 0x0C010C00u);
  u32x4 d;
  d[0] = y & 0x00030003u;
  d[1] = (y >> 2) & 0x00030003u;
  d[2] = (y >> 4) & 0x00030003u;
  d[3] = (y >> 6) & 0x00030003u;
  return d;
}
// 4-bit: the field is the whole word.
__device__ __forceinline__ u32x4 unpack4(uint32_t w) {
  u32x4 d;
  d[0] = w & 0x000F000Fu;
  d[1] = (w >> 4) & 0x000F000Fu;
  d[2] = (w >> 8) & 0x000F000Fu;
  d[3] = (w >> 12) & 0x000F000Fu;
  return d;
}
// 8-bit: codes 0..3 in lo, 4..7 in hi.
__device__ __forceinline__ u32x4 unpack8(uint32_t lo, uint32_t hi) {
  u32x4 d;
#pragma unroll
  for (int m = 0; m < 4; ++m) d[m] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u + uint32_t(m) * 0x00010001u);
  return d;
}

// x[8] -> hi + lo fp16 parts in the same dword order (x_m, x_m+4)
__device__ __forceinline__ void split_hi_lo(const float (&x)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(x[m], x[m + 4]);
    const float r0 = x[m] - float(h[0]);
    const float r1 = x[m + 4] - float(h[1]);
    const auto l = __builtin_amdgcn_cvt_pkrtz(r0, r1);
    hi[m] = __builtin_bit_cast(uint32_t, h);
    lo[m] = __builtin_bit_cast(uint32_t, l);
  }
}

__device__ __forceinline__ void load_f16x8(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = h2f(uint16_t(w[k] & 0xFFFFu));
    v[2 * k + 1] = h2f(uint16_t(w[k] >> 16));
  }
}

template <int NB>  // load NB bytes (2, 4, 8, 16, 32 or 64) into words
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

template <int BITS, int NW>
__device__ __forceinline__ u32x4 codes8(const uint32_t (&w)[NW], int idx) {
  // field idx of 8*BITS bits inside the loaded words
  if constexpr (BITS == 2) return unpack2(w[idx >> 1], idx & 1);
  else if constexpr (BITS == 4) return unpack4(w[idx]);
  else return unpack8(w[2 * idx], w[2 * idx + 1]);
}

template <int G, int DK, int DV, int KB, int VB>
__global__ __launch_bounds__(kDecodeThreads) void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int KK = DK / 32;          // score k-steps (32 channels each)
  constexpr int NV = DV / 16;          // value tiles (16 channels each)
  constexpr int NGV = DV / 32;         // value channel groups
  constexpr int KLB = DK * KB / 32;    // key-row bytes per lane (a quarter row)
  constexpr int KLW = KLB < 4 ? 1 : KLB / 4;
  constexpr int VLB = 2 * VB;          // value bytes per lane per channel group (2 channels x 8 tokens)
  constexpr int VLW = VLB < 4 ? 1 : VLB / 4;
  constexpr int NT = 2 * G;            // MFMA columns / rows in use
  constexpr int BPQ = DK / 8;          // 8-channel blocks per query
  constexpr int QTASKS = G * BPQ;
  constexpr int QR = (QTASKS + 63) / 64;
  constexpr int NZ = (NGV + 1) / 2;    // value channel groups per P' lane
  static_assert(NT <= 16 && DK % 32 == 0 && DV % 32 == 0 && DK <= 256 && DV <= 256, "shape");
  static_assert(BPQ <= 64, "bias reduction assumes a query's blocks fit one wave");

  extern __shared__ __align__(16) unsigned char smem[];
  float* qs_lds = reinterpret_cast<float*>(smem);                   // [G][DK] scale*log2e*q
  float* qexp = qs_lds + G * DK;                                    // [G] 2^-E per query
  constexpr int kHead = ((G * DK + G) * 4 + 15) / 16 * 16;
  constexpr int kWaveBytes = (KK + NGV) * 64 * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, gq = lane >> 4;
  u32x4* QB = reinterpret_cast<u32x4*>(smem + kHead + wave * kWaveBytes);   // [KK][4][16]
  u32x4* PA = QB + KK * 64;                                                 // [NGV][4][16]

  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nG = a.L.n_groups, R = a.L.R, P = a.P, Tq = a.L.Tq;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  const int g0 = int(int64_t(p) * nG / P), g1 = int(int64_t(p + 1) * nG / P);
  const int r0 = int(int64_t(p) * R / P), r1 = int(int64_t(p + 1) * R / P);

  // ---------------------------------------------------------------- set-up
  for (int idx = tid; idx < G * DK; idx += kDecodeThreads)
    qs_lds[idx] = a.scale * kLog2e * load_q_any(a.q, a.q_dtype, (int64_t(b) * a.L.Hq + int64_t(h) * G) * DK + idx);
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int k = lane; k < (KK + NGV) * 64; k += 64) QB[k] = zero;
  }
  __syncthreads();
  if (wave == 0) {
    // per query: 2^-E with E >= 0 the smallest exponent such that |q * 2^-E| <= 1,
    // keeping q_c s_c inside the fp16 range
    for (int i = 0; i < G; ++i) {
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

  // compact Q' tasks of this lane: query ti, 8-channel block tb
  float qsv[QR][8];
  int ti[QR], tb[QR];
#pragma unroll
  for (int rr = 0; rr < QR; ++rr) {
    const int tau = lane + 64 * rr;
    ti[rr] = tau < QTASKS ? tau / BPQ : 0;
    tb[rr] = tau % BPQ;
#pragma unroll
    for (int k = 0; k < 8; ++k) qsv[rr][k] = 0.0f;
    if (tau < QTASKS) {
#pragma unroll
      for (int k = 0; k < 8; ++k) qsv[rr][k] = qs_lds[ti[rr] * DK + 8 * tb[rr] + k] * qexp[ti[rr]];
    }
  }
  // this lane's column / row in the MFMA tiles: query iD, part (hi/lo) = n & 1
  const int iD = n >> 1;
  const bool dvalid = n < NT;
  const float qe = dvalid ? qexp[iD] : 1.0f;
  const float coefD = 16777216.0f / qe;  // 2^24 * 2^E
  const float coefB = 1.0f / qe;         // 2^E

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 oacc[NV];
#pragma unroll
  for (int t = 0; t < NV; ++t) oacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float zacc[NZ];
#pragma unroll
  for (int k = 0; k < NZ; ++k) zacc[k] = 0.0f;

  const uint8_t* kcodes = static_cast<const uint8_t*>(a.cache.k_codes);
  const uint16_t* kscale = static_cast<const uint16_t*>(a.cache.k_scale);
  const uint16_t* kzero = static_cast<const uint16_t*>(a.cache.k_zero);
  const uint8_t* vcodes = static_cast<const uint8_t*>(a.cache.v_codes);
  const uint16_t* vscale = static_cast<const uint16_t*>(a.cache.v_scale);
  const uint16_t* vzero = static_cast<const uint16_t*>(a.cache.v_zero);

  // ------------------------------------------------------------ key groups
  for (int g = g0 + wave; g < g1; g += kDecodeWaves) {
    const int64_t gg = slab * nG + g;
    // key codes of the two 16-token tiles: tile tt row n is token 8(n/4) + 4tt + n%4
    uint32_t kw[2][KLW];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = 8 * (n >> 2) + 4 * tt + (n & 3);
      load_bytes<KLB>(kcodes + ((slab * Tq + int64_t(g) * KVQ_GROUP + tok) * (DK * KB / 8)) + gq * KLB, kw[tt]);
    }
    // value codes: channel group gc, channels 32gc + 2n, +1, tokens 8gq..8gq+7
    uint32_t vw[NGV][VLW];
#pragma unroll
    for (int gc = 0; gc < NGV; ++gc)
      load_bytes<VLB>(vcodes + ((gg * 4 + gq) * DV + 32 * gc + 2 * n) * VB, vw[gc]);

    // Q' = q s (hi, lo) for the compact tasks, and the zero-point bias partials
    float bpart[QR];
#pragma unroll
    for (int rr = 0; rr < QR; ++rr) {
      bpart[rr] = 0.0f;
      if (lane + 64 * rr < QTASKS) {
        float s8[8], z8[8], x[8];
        load_f16x8(kscale + gg * DK + 8 * tb[rr], s8);
        load_f16x8(kzero + gg * DK + 8 * tb[rr], z8);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          x[k] = qsv[rr][k] * s8[k];
          bpart[rr] = fmaf(qsv[rr][k], z8[k], bpart[rr]);
        }
        u32x4 hi, lo;
        split_hi_lo(x, hi, lo);
        const int kk = tb[rr] % KK, gqb = tb[rr] / KK;
        QB[(kk * 4 + gqb) * 16 + 2 * ti[rr]] = hi;
        QB[(kk * 4 + gqb) * 16 + 2 * ti[rr] + 1] = lo;
      }
#pragma unroll
      for (int off = 1; off < BPQ; off <<= 1) bpart[rr] += __shfl_xor(bpart[rr], off, 64);
    }
    // bias of this lane's query: held by lane (iD * BPQ) % 64 of round (iD * BPQ) / 64
    float bias = 0.0f;
#pragma unroll
    for (int rr = 0; rr < QR; ++rr) {
      const float v = __shfl(bpart[rr], (iD * BPQ) & 63, 64);
      if ((iD * BPQ) / 64 == rr) bias = v;
    }
    wave_lds_sync();

    // scores
    f32x4 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 A = codes8<KB>(kw[tt], kk);
        const u32x4 Bq = QB[(kk * 4 + gq) * 16 + n];
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(A), as_half8(Bq), sacc[tt], 0, 0, 0);
      }
    }
    // lane (n, gq): tile tt, row r -> token 8gq + 4tt + r, column n = (query iD, part n&1)
    float sv[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sacc[tt][r];
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // + other part
        v = fmaf(v, coefD, bias * coefB);
        sv[4 * tt + r] = v;
        mloc = fmaxf(mloc, v);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    if (__any(dvalid && m_new > m_run)) {  // rescale (rare once the running maxima settle)
      const float alpha = lse_weight(m_run, m_new);
      l_run *= alpha;
#pragma unroll
      for (int k = 0; k < NZ; ++k) zacc[k] *= alpha;
      // value rows 4gq + r are (query 2gq + r/2, part r&1): fetch their alphas
      const float a0 = __shfl(alpha, 16 * gq + 4 * gq, 64);
      const float a1 = __shfl(alpha, 16 * gq + 4 * gq + 2, 64);
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        oacc[t][0] *= a0;
        oacc[t][1] *= a0;
        oacc[t][2] *= a1;
        oacc[t][3] *= a1;
      }
      m_run = m_new;
    }
    float pv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pv[k] = exp2f(sv[k] - m_run);
      l_run += pv[k];
    }

    // P' = p s (hi, lo) for this lane's channel groups gc = n&1, n&1 + 2, ...
    if (dvalid) {
#pragma unroll
      for (int k2 = 0; k2 < NZ; ++k2) {
        const int gc = (n & 1) + 2 * k2;
        if (gc < NGV) {
          float s8[8], z8[8], x[8];
          load_f16x8(vscale + (gg * NGV + gc) * KVQ_GROUP + 8 * gq, s8);
          load_f16x8(vzero + (gg * NGV + gc) * KVQ_GROUP + 8 * gq, z8);
          float zs = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            x[k] = pv[k] * s8[k];
            zs = fmaf(pv[k], z8[k], zs);
          }
          zacc[k2] += zs;
          u32x4 hi, lo;
          split_hi_lo(x, hi, lo);
          PA[(gc * 4 + gq) * 16 + 2 * iD] = hi;
          PA[(gc * 4 + gq) * 16 + 2 * iD + 1] = lo;
        }
      }
    }
    wave_lds_sync();

    // values
#pragma unroll
    for (int gc = 0; gc < NGV; ++gc) {
      const u32x4 Ap = PA[(gc * 4 + gq) * 16 + n];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const u32x4 Bv = codes8<VB>(vw[gc], half);
        oacc[2 * gc + half] =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(Ap), as_half8(Bv), oacc[2 * gc + half], 0, 0, 0);
      }
    }
    wave_lds_sync();
  }

  // ----------------------------------------------- retained fp16 rows (VALU)
  // state kept separately: m_r, l_r wave-uniform, o_r over channels lane + 64 j
  constexpr int RJ = (DV + 63) / 64;
  float m_r[G], l_r[G], o_r[G][RJ];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m_r[i] = -INFINITY;
    l_r[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < RJ; ++j) o_r[i][j] = 0.0f;
  }
  {
    float* pp = reinterpret_cast<float*>(PA);  // [32][G] probabilities of the chunk
    const int t = lane & 31, hf = lane >> 5;
    const int nchunks = (r1 - r0 + KVQ_GROUP - 1) / KVQ_GROUP;
    for (int ck = wave; ck < nchunks; ck += kDecodeWaves) {
      const int rbeg = r0 + ck * KVQ_GROUP, r = rbeg + t;
      const bool valid = r < r1;
      float acc[G];
#pragma unroll
      for (int i = 0; i < G; ++i) acc[i] = 0.0f;
      if (valid) {
        const uint16_t* krow = static_cast<const uint16_t*>(a.cache.k_fp16) + (slab * R + r) * DK;
        for (int c = hf * (DK / 2); c < (hf + 1) * (DK / 2); ++c) {
          const float kv = h2f(krow[c]);
#pragma unroll
          for (int i = 0; i < G; ++i) acc[i] = fmaf(qs_lds[i * DK + c], kv, acc[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float s = valid ? acc[i] + __shfl_xor(acc[i], 32, 64) : -INFINITY;
        float mx = s;
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
        const float mn = fmaxf(m_r[i], mx);
        const float al = lse_weight(m_r[i], mn);
        const float pr = valid ? exp2f(s - mn) : 0.0f;
        float ps = pr;
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) ps += __shfl_xor(ps, m, 64);
        l_r[i] = l_r[i] * al + ps;
        m_r[i] = mn;
#pragma unroll
        for (int j = 0; j < RJ; ++j) o_r[i][j] *= al;
        if (hf == 0) pp[t * G + i] = pr;
      }
      wave_lds_sync();
      const int nrow = r1 - rbeg < KVQ_GROUP ? r1 - rbeg : KVQ_GROUP;
      for (int tt = 0; tt < nrow; ++tt) {
        const uint16_t* vrow = static_cast<const uint16_t*>(a.cache.v_fp16) + (slab * R + rbeg + tt) * DV;
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
          const int c = lane + 64 * j;
          if (c < DV) {
            const float vv = h2f(vrow[c]);
#pragma unroll
            for (int i = 0; i < G; ++i) o_r[i][j] = fmaf(pp[tt * G + i], vv, o_r[i][j]);
          }
        }
      }
      wave_lds_sync();
    }
  }

  // -------------------------------------------- combine the 8 wave states
  __syncthreads();  // every wave is out of its loops; per-wave LDS is free now
  float* st = reinterpret_cast<float*>(smem + kHead);   // [8][G][DV + 2]
  float* zb = st + 8 * G * (DV + 2);                      // [4][G][NGV]
  float* res = zb + 4 * G * NGV;                          // [G][DV + 2]
  int* flag = reinterpret_cast<int*>(res + G * (DV + 2));
  {
    float* s0 = st + (2 * wave) * G * (DV + 2);
    // matrix-core state: m from lane (2i, gq 0), l summed over lane groups
    const float l_all = l_run + __shfl_xor(l_run, 16, 64) + __shfl_xor(l_run, 32, 64) +
                        __shfl_xor(__shfl_xor(l_run, 16, 64), 32, 64);
    if (gq == 0 && dvalid && (n & 1) == 0) {
      s0[iD * (DV + 2)] = m_run;
      s0[iD * (DV + 2) + 1] = l_all;
    }
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int c = 32 * (t >> 1) + 2 * n + (t & 1);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int i = 2 * gq + half;
        if (i < G) s0[i * (DV + 2) + 2 + c] = 16777216.0f * (oacc[t][2 * half] + oacc[t][2 * half + 1]);
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < NZ; ++k2) {
      float z = zacc[k2] + __shfl_xor(zacc[k2], 16, 64);
      z += __shfl_xor(z, 32, 64);
      const int gc = (n & 1) + 2 * k2;
      if (gq == 0 && dvalid && gc < NGV) zb[(wave * G + iD) * NGV + gc] = z;
    }
    // retained state
    float* s1 = st + (2 * wave + 1) * G * (DV + 2);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (lane == 0) {
        s1[i * (DV + 2)] = m_r[i];
        s1[i * (DV + 2) + 1] = l_r[i];
      }
#pragma unroll
      for (int j = 0; j < RJ; ++j) {
        const int c = lane + 64 * j;
        if (c < DV) s1[i * (DV + 2) + 2 + c] = o_r[i][j];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * DV; idx += kDecodeThreads) {
    const int i = idx / DV, c = idx - i * DV;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; ++s) M = fmaxf(M, st[(s * G + i) * (DV + 2)]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float* e = st + (s * G + i) * (DV + 2);
      const float w = lse_weight(e[0], M);
      L += w * e[1];
      float v = e[2 + c];
      if ((s & 1) == 0) v += zb[((s >> 1) * G + i) * NGV + c / 32];
      O += w * v;
    }
    res[i * (DV + 2) + 2 + c] = O;
    if (c == 0) {
      res[i * (DV + 2)] = M;
      res[i * (DV + 2) + 1] = L;
    }
  }
  __syncthreads();
  finish_partition(a, G, b, h, p, res, flag);
}

template <int G, int DK, int DV, int KB, int VB>
hipError_t launch_one(const DecodeArgs& a, hipStream_t stream) {
  constexpr int KK = DK / 32, NGV = DV / 32;
  constexpr size_t head = ((G * DK + G) * 4 + 15) / 16 * 16;
  constexpr size_t loop = head + size_t(kDecodeWaves) * (KK + NGV) * 64 * 16;
  constexpr size_t merge = head + (8 * G * (DV + 2) + 4 * G * NGV + G * (DV + 2) + 4) * 4;
  constexpr size_t lds = loop > merge ? loop : merge;
  static_assert(lds <= 64 * 1024, "LDS budget");
  const dim3 grid(unsigned(a.P), unsigned(a.L.Hkv), unsigned(a.L.B));
  hipLaunchKernelGGL((decode_mfma_kernel<G, DK, DV, KB, VB>), grid, dim3(kDecodeThreads), lds, stream, a);
  return hipGetLastError();
}

template <int G, int DK, int DV>
hipError_t launch_bits(const DecodeArgs& a, hipStream_t stream) {
  const int kb = a.L.k_bits, vb = a.L.v_bits;
#define KVQ_BITS_CASE(K_, V_) \
  if (kb == K_ && vb == V_) return launch_one<G, DK, DV, K_, V_>(a, stream);
  KVQ_BITS_CASE(2, 2) KVQ_BITS_CASE(2, 4) KVQ_BITS_CASE(2, 8)
  KVQ_BITS_CASE(4, 2) KVQ_BITS_CASE(4, 4) KVQ_BITS_CASE(4, 8)
  KVQ_BITS_CASE(8, 2) KVQ_BITS_CASE(8, 4) KVQ_BITS_CASE(8, 8)
#undef KVQ_BITS_CASE
  return hipErrorNotSupported;
}

template <int DK, int DV>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  switch (a.L.Hq / a.L.Hkv) {
    case 1: return launch_bits<1, DK, DV>(a, stream);
    case 4: return launch_bits<4, DK, DV>(a, stream);
    case 8: return launch_bits<8, DK, DV>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const int Dk = a.L.Dk, Dv = a.L.Dv;
  if (Dk == 128 && Dv == 128) return launch_g<128, 128>(a, stream);
  if (Dk == 32 && Dv == 128) return launch_g<32, 128>(a, stream);
  if (Dk == 64 && Dv == 64) return launch_g<64, 64>(a, stream);
  return hipErrorNotSupported;
}

}  // namespace kvq
