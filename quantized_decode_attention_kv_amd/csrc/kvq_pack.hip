// kv_quant_pack kernel for gfx950.
//
// Group-wise asymmetric min/max quantization with fp16 scale/zero: keys per
// channel over 32 consecutive quantized tokens ("LogQuant: Log-Distributed 2-Bit
// Quantization of KV Cache", section 5, per-channel keys; group 32 from "Quantize
// What Counts: More for Keys, Less for Values", results), values per token over
// v_group = 32, 64 or 128 channels (the group sizes that page's results sweep),
// separate key / value bit widths (Quantize What Counts, methodology).
// Retained positions (LogQuant section 2) are copied to fp16 rows.
//
// One launch per call (two when key groups span 64 or 128 tokens: key_range_kernel
// first forms their scales and zeros).  Heads of 128 channels with 16-bit inputs
// and 32-token key groups take pack128_kernel (described at its definition); the
// rest take pack_kernel.  With key rotation (KVQ_KEY_ROTATION) every key row is
// rotated in float32 before its min / max, codes or fp16 copy.
// pack_kernel: workgroups [0, n_groups_chunk) each own one key group of
// one (batch, kv-head) slab; the remaining workgroups copy the chunk's retained
// rows to fp16.  In a group workgroup, wave w holds tokens 8w..8w+7 and lane l the
// channel pair (2l, 2l+1) (and 2l+128, 2l+129 for heads wider than 128), so every
// global load is a coalesced row segment:
//   keys    per-channel min / max over the wave's 8 tokens in registers, across
//           the 4 waves through LDS;
//   values  per-(token, v_group-channel group) min / max with DPP reductions
//           over the lanes that hold the group (v_group = 32, 64 or 128);
//   codes   placed into LDS words at their final bit positions (a lane's two
//           4- or 8-bit key codes fill whole bytes and are stored plainly; 2-bit
//           key codes and value codes are OR-ed in), then stored as one
//           contiguous run per group.
//
// The codes follow the quantizer contract of kvq.h bit for bit: code =
// clamp(rint(fl(x - z) / s)) with the correctly rounded division.  The division is
// replaced by a multiply with r, the hardware reciprocal of s (within one ulp):
// the product and the correctly rounded quotient differ by at most
// 4 * 2^-24 * |t| (< 1.3e-4 while |t| <= 512, and t stays below 2 * (2^bits - 1)
// because s is at least about half of range / levels; larger t clamp the same
// way), so rint gives the same integer unless the quotient lies within 2^-12 of a
// half-integer; such elements (about one in two thousand) take the exact division.
// Scale and zero use the exact division, with contraction off, as the contract
// spells out.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.hpp"
#include "kvq_retention.hpp"
#include "kvq_rotate.hpp"
#include "kvq_vlayout.hpp"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackWaves = kPackThreads / 64;
constexpr int kRetRowsPerBlock = 4;
constexpr int kRetRows128 = 32;  // retained rows per workgroup of pack128_kernel
constexpr int kMaxPairBlocks = KVQ_MAX_HEAD_DIM / 128;  // 64-lane blocks of channel pairs

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<KVQ_F32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_elem<KVQ_F16>(const void* p, int64_t i) {
  return __half2float(static_cast<const __half*>(p)[i]);
}
template <>
__device__ __forceinline__ float load_elem<KVQ_BF16>(const void* p, int64_t i) {
  return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
}

// elements i, i + 1 (i even) as fp32
template <int DT>
__device__ __forceinline__ float2 load_pair(const void* p, int64_t i) {
  if constexpr (DT == KVQ_F32) {
    return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
    if constexpr (DT == KVQ_BF16) {
      return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
    } else {
      return make_float2(__half2float(__ushort_as_half(uint16_t(w & 0xFFFFu))),
                         __half2float(__ushort_as_half(uint16_t(w >> 16))));
    }
  }
}

// 16 consecutive elements starting at i (16 * element size bytes, aligned) as
// raw words (f32: 16 words; 16-bit types: 8 words), converted by cvt16
template <int DT>
struct Raw16 {
  static constexpr int kWords = DT == KVQ_F32 ? 16 : 8;
  uint32_t w[kWords];
};
template <int DT>
__device__ __forceinline__ Raw16<DT> load16(const void* p, int64_t i) {
  Raw16<DT> r;
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(p) + i * (DT == KVQ_F32 ? 4 : 2));
#pragma unroll
  for (int k = 0; k < Raw16<DT>::kWords / 4; ++k) {
    const uint4 v = src[k];
    r.w[4 * k] = v.x;
    r.w[4 * k + 1] = v.y;
    r.w[4 * k + 2] = v.z;
    r.w[4 * k + 3] = v.w;
  }
  return r;
}
template <int DT>
__device__ __forceinline__ void cvt16(const Raw16<DT>& r, float (&x)[16]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if constexpr (DT == KVQ_F32) {
      x[2 * k] = __uint_as_float(r.w[2 * k]);
      x[2 * k + 1] = __uint_as_float(r.w[2 * k + 1]);
    } else if constexpr (DT == KVQ_BF16) {
      x[2 * k] = __uint_as_float(r.w[k] << 16);
      x[2 * k + 1] = __uint_as_float(r.w[k] & 0xFFFF0000u);
    } else {
      x[2 * k] = __half2float(__ushort_as_half(uint16_t(r.w[k] & 0xFFFFu)));
      x[2 * k + 1] = __half2float(__ushort_as_half(uint16_t(r.w[k] >> 16)));
    }
  }
}

__device__ __forceinline__ uint16_t f16_bits_rne(float x) {
  return __half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

struct QParams {
  float s, z, r;  // scale and zero (their fp16 values) and fl(1/s) (0 when s == 0)
  uint16_t s_bits, z_bits;
};

// fl(a / L), correctly rounded, for a level count L = 2^b - 1 (b in {1, 2, 3, 4, 8})
// and any non-negative finite a, without a divide: q0 = a * fl(1/L) and one
// fma-corrected step (Markstein's correction with an exact residual).  Checked
// against the correctly rounded quotient for every non-negative finite float and
// each of those five L: bit-identical.  fl(1/L) folds to a constant where L is one.
// The result is kept opaque so that its fp16 conversion cannot be fused into the
// last fma (one rounding of the exact value instead of two).
__device__ __forceinline__ float quotient_by_levels(float a, float L) {
  const float y = 1.0f / L;
  const float q0 = a * y;
  const float r = fmaf(-q0, L, a);
  float q = fmaf(r, y, q0);
  asm("" : "+v"(q));
  return q;
}

// s = fp16(fp32(mx - mn) / (2^bits - 1)), z = fp16(mn); zeros stored as +0.
__device__ __forceinline__ QParams make_qparams(float mn, float mx, float levels) {
  const float range = mx - mn;
  const float s32 = quotient_by_levels(range, levels);
  uint16_t sb = f16_bits_rne(s32);
  uint16_t zb = f16_bits_rne(mn);
  if ((sb & 0x7fffu) == 0) sb = 0;
  if ((zb & 0x7fffu) == 0) zb = 0;
  QParams q;
  q.s_bits = sb;
  q.z_bits = zb;
  q.s = f16_bits_to_f32(sb);
  q.z = f16_bits_to_f32(zb);
  q.r = q.s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(q.s);
  return q;
}

// the same parameters from stored fp16 bits (key groups longer than 32 tokens)
__device__ __forceinline__ QParams qparams_of(uint16_t sb, uint16_t zb) {
  QParams q;
  q.s_bits = sb;
  q.z_bits = zb;
  q.s = f16_bits_to_f32(sb);
  q.z = f16_bits_to_f32(zb);
  q.r = q.s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(q.s);
  return q;
}

// log2(k_group / 32): key group of code group g is g >> key_group_shift
__device__ __host__ __forceinline__ int key_group_shift(int k_group) {
  return k_group == 128 ? 2 : (k_group == 64 ? 1 : 0);
}

// code = 0 if s == 0 else clamp(rint(fl(x - z) / s), 0, levels) (see the header)
__device__ __forceinline__ uint32_t quant_code(float x, float s, float z, float r, float levels) {
  const float u = x - z;
  float t = u * r;  // s == 0: r == 0, t == 0, code 0
  float rt = __builtin_rintf(t);
  if (__builtin_expect(fabsf(t - rt) > 0.5f - 1.0f / 4096.0f, 0)) {
    t = u / s;
    rt = __builtin_rintf(t);
  }
  rt = fminf(fmaxf(rt, 0.0f), levels);
  return uint32_t(rt);
}

// quant_code for N elements with one check: when no element's fast quotient lies
// within 2^-12 of a half-integer (the usual case) no element takes the division, and
// the wave tests that once instead of once per element.  The codes come back as
// exact integers held in floats (clamped with one med3).
template <int N>
__device__ __forceinline__ void quant_levels(const float (&x)[N], const float (&s)[N], const float (&z)[N],
                                             const float (&r)[N], float levels, float (&code)[N]) {
  float u[N], rt[N];
  float worst = 0.0f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    u[k] = x[k] - z[k];
    const float t = u[k] * r[k];  // s == 0: r == 0, t == 0, code 0
    rt[k] = __builtin_rintf(t);
    worst = fmaxf(worst, fabsf(t - rt[k]));
  }
  if (__builtin_expect(worst > 0.5f - 1.0f / 4096.0f, 0)) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const float t = u[k] * r[k];
      if (fabsf(t - rt[k]) > 0.5f - 1.0f / 4096.0f) rt[k] = __builtin_rintf(u[k] / s[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < N; ++k) code[k] = __builtin_amdgcn_fmed3f(rt[k], 0.0f, levels);
}

// quant_levels with one fma per element for the fast quotient: t = fl(x r + nzr),
// nzr = fl(-z r), r = rcp(s) (one ulp).  Against the contract's V = fl(fl(x - z) / s),
// |t - V| <= |Q| 2^-21.6 + |z r| 2^-23.9 with Q = (x - z) / s (rounding of the fma,
// of nzr and of the reciprocal, and the contract's own two roundings); where
// |Q| > levels + 1 both sides clamp to the same code, so with |Q| <= 256 the bound
// delta = 2^-13 + |z r| 2^-23 holds, and an element whose t lies within
// lim = 0.5 - delta of an integer gets the same code as V (|V - rint(t)| < 0.5).
// The others (near-ties; rare) take the division.  nzr_max: the largest |nzr| of
// the elements; s == 0 gives r == 0, t = -0 or +0 and code 0, as the contract says.
// exact(k) returns fl(fl(x_k - z_k) / s_k) (the contract's quotient; called rarely).
__device__ __forceinline__ float fma_quant_limit(float nzr_max) {
  return 0.5f - (0x1p-13f + nzr_max * 0x1p-23f);
}
//
// clamp (wave-uniform) false skips the clamp to [0, levels]; the caller passes
// false only when every element's group has |z r| <= 128 and s >= 2^-14 (r <=
// 2^14) or s == 0 (clamp_free below), where the contract's clamp changes nothing:
// with z = fp16(mn), |mn - z| <= 2^-11 |mn| (or <= 2^-25 for fp16-subnormal mn),
// so (x - z) / s >= -2^-11 |z| / s >= -0.07; and s >= fl(fl(mx - mn) / levels)
// (1 - 2^-11), so (x - z) / s <= levels (1 + 2^-10.9) + 0.07 < levels + 0.5.
// Both round into [0, levels] (a -0 code converts to 0).
__device__ __forceinline__ bool clamp_free(float nzr_max, float r_max) {
  return nzr_max <= 128.0f && r_max <= 16384.0f;
}
template <int N, typename Exact>
__device__ __forceinline__ void quant_levels_fma(const float (&x)[N], const float (&r)[N], const float (&nzr)[N],
                                                 float lim, float levels, bool clamp, float (&code)[N],
                                                 Exact&& exact) {
  float t[N], rt[N];
  float worst = 0.0f;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    t[k] = fmaf(x[k], r[k], nzr[k]);
    rt[k] = __builtin_rintf(t[k]);
    worst = fmaxf(worst, fabsf(t[k] - rt[k]));
  }
  if (__builtin_expect(worst > lim, 0)) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (fabsf(t[k] - rt[k]) > lim) rt[k] = __builtin_rintf(exact(k));
    }
  }
  if (clamp) {
#pragma unroll
    for (int k = 0; k < N; ++k) rt[k] = __builtin_amdgcn_fmed3f(rt[k], 0.0f, levels);
  }
#pragma unroll
  for (int k = 0; k < N; ++k) code[k] = rt[k];
}

// Byte `b` of `w` replaced by the code q (an integer in [0, 255] held as a float,
// so the conversion is exact whatever its rounding): one instruction that both
// converts and places the code.
__device__ __forceinline__ uint32_t put_byte(float q, uint32_t b, uint32_t w) {
  return __builtin_amdgcn_cvt_pk_u8_f32(q, b, w);
}

// Every output of the pack is written with streaming (non-temporal) stores: the
// packed cache is read next by decode, a whole cache later, so there is no point in
// keeping the freshly written lines in the caches, where their write-back would
// fall into that decode's read stream.  (A plain 32 MB fill right before the 128K
// decode cost the decode 13 us with ordinary stores and nothing with streaming
// ones; for this kernel's 35 MB the two measured the same, within noise.)
template <typename T>
__device__ __forceinline__ void out_store(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}

// The DPP exchanges below (quad permutations and row mirrors, all rows and banks
// enabled) read a lane of the same row that always exists, so bound_ctrl changes
// nothing about their results; it is set so that the compiler can fold the
// exchange into the ALU instruction that consumes it (one instruction instead of a
// move and the operation).
// min / max over the 16 lanes of a DPP row (every lane gets the result)
template <bool MAX>
__device__ __forceinline__ float row16_reduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));   // quad_perm 1,0,3,2
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));   // quad_perm 2,3,0,1
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));  // row_half_mirror
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));  // row_mirror
  return v;
}

// OR a B-bit code into LDS words at stream bit `bit`; a 3-bit code may straddle
// into the next word (other widths never do)
template <int B>
__device__ __forceinline__ void or_code(uint32_t* w, int bit, uint32_t code) {
  const int sh = bit & 31;
  atomicOr(&w[bit >> 5], code << sh);
  if constexpr (B == 3) {
    if (sh > 32 - B) atomicOr(&w[(bit >> 5) + 1], code >> (32 - sh));
  }
}

// Key rotation of the wave's 8 rows as pack_kernel holds them: channels 2cp and
// 2cp + 1 of pair block k (cp = lane + 64k) in x[k][t].x / .y, so channel bit 0 is
// the pair, bits 1 .. 6 the lane and bits 7 .. the block.  Butterfly h = 1 in the
// pair, 2 .. 64 with lane ^ h/2, 128 and up across blocks, in increasing h; lanes
// past the row hold zeros and meet only each other.
template <int P>
__device__ __forceinline__ void rotate_pair_rows(float2 (&x)[P][8], int lane, int Dk) {
#pragma unroll
  for (int k = 0; k < P; ++k) {
    if (128 * k >= Dk) break;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float u = x[k][t].x, v = x[k][t].y;
      x[k][t] = make_float2(u + v, u - v);
    }
  }
  for (int hl = 1; hl < 64 && 2 * hl < Dk; hl <<= 1) {
    const bool upper = (lane & hl) != 0;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if (128 * k >= Dk) break;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        x[k][t].x = butterfly(x[k][t].x, __shfl_xor(x[k][t].x, hl), upper);
        x[k][t].y = butterfly(x[k][t].y, __shfl_xor(x[k][t].y, hl), upper);
      }
    }
  }
#pragma unroll
  for (int hk = 1; hk < P; hk <<= 1) {
    if (128 * hk >= Dk) break;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if ((k & hk) || 128 * (k + hk) >= Dk) continue;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float2 u = x[k][t], v = x[k + hk][t];
        x[k][t] = make_float2(u.x + v.x, u.y + v.y);
        x[k + hk][t] = make_float2(u.x - v.x, u.y - v.y);
      }
    }
  }
  const float sc = rotation_scale(31 - __builtin_clz(unsigned(Dk)));
#pragma unroll
  for (int k = 0; k < P; ++k) {
#pragma unroll
    for (int t = 0; t < 8; ++t) x[k][t] = make_float2(rotation_scaled(x[k][t].x, sc), rotation_scaled(x[k][t].y, sc));
  }
}

template <int DT, int KB, int VB>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const PackArgs a) {
  __shared__ int32_t row_s[KVQ_GROUP];
  __shared__ float kmn_s[kPackWaves][KVQ_MAX_HEAD_DIM], kmx_s[kPackWaves][KVQ_MAX_HEAD_DIM];
  __shared__ float ks_s[KVQ_MAX_HEAD_DIM], kz_s[KVQ_MAX_HEAD_DIM], kr_s[KVQ_MAX_HEAD_DIM];
  __shared__ uint32_t kw_s[KVQ_GROUP * KVQ_MAX_HEAD_DIM * KB / 32];  // key code words of the group
  __shared__ uint32_t vw_s[KVQ_MAX_HEAD_DIM * VB];                   // value code stream of the group
  __shared__ uint16_t vs_s[KVQ_MAX_HEAD_DIM / KVQ_GROUP][KVQ_GROUP], vz_s[KVQ_MAX_HEAD_DIM / KVQ_GROUP][KVQ_GROUP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int Dk = a.L.Dk, Dv = a.L.Dv;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  const RetentionRule rr{a.L.T, a.L.n_recent, a.L.log_window};

  if (int64_t(blockIdx.x) < a.n_groups_chunk) {
    // ------------------------------------------------ one key group of 32 tokens
    const int64_t g = a.g_begin + blockIdx.x;
    const int kwords = Dk * KB / 32, vwords = Dv * VB;
    // rows of the wave's 8 tokens in the chunk: a group wholly below the first
    // retained position holds positions 32g .. 32g + 31 (one closed-form count
    // decides it); otherwise each token's position comes from the search
    const bool plain = quantized_before(rr, (g + 1) * KVQ_GROUP) == (g + 1) * KVQ_GROUP;
    if (!plain) {
      if (tid < KVQ_GROUP) row_s[tid] = int32_t(quantized_position(rr, g * KVQ_GROUP + tid) - a.t_begin);
      __syncthreads();
    }
    auto row_of = [&](int tok) -> int32_t {
      return plain ? int32_t(g * KVQ_GROUP + tok - a.t_begin) : row_s[tok];
    };
    int32_t rows[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) rows[t] = row_of(8 * wave + t);
    // Dv == 128: thread (token tid / 8, 16-channel tile tid % 8) takes its value
    // row segment now, so that its load latency overlaps the key phase
    const bool v128 = Dv == 128 && VB >= 2 && VB != 3;  // 1- and 3-bit values take the generic path
    const int vtok = tid >> 3, vtile = tid & 7;
    Raw16<DT> vraw;
    if (v128) vraw = load16<DT>(a.V, (slab * a.t_count + row_of(vtok)) * 128 + 16 * vtile);

    // (4- and 8-bit key words are written byte by byte below, every byte once)
    if constexpr (KB <= 3) {
      for (int i = tid; i < KVQ_GROUP * kwords; i += kPackThreads) kw_s[i] = 0u;
    }
    for (int i = tid; i < vwords; i += kPackThreads) vw_s[i] = 0u;

    // keys: lane holds channels (2cp, 2cp+1) of the wave's 8 tokens; per-channel
    // min / max over them, then across waves
    constexpr float k_levels = float((1 << KB) - 1);
    float2 kx[kMaxPairBlocks][8];
#pragma unroll
    for (int k = 0; k < kMaxPairBlocks; ++k) {
      const int cp = lane + 64 * k;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        kx[k][t] = 2 * cp < Dk ? load_pair<DT>(a.K, (slab * a.t_count + rows[t]) * Dk + 2 * cp) : make_float2(0.0f, 0.0f);
    }
    if (a.L.flags & KVQ_KEY_ROTATION) rotate_pair_rows(kx, lane, Dk);
#pragma unroll
    for (int k = 0; k < kMaxPairBlocks; ++k) {
      const int cp = lane + 64 * k;
      if (2 * cp < Dk) {
        float2 mn = kx[k][0], mx = kx[k][0];
#pragma unroll
        for (int t = 1; t < 8; ++t) {
          mn = make_float2(fminf(mn.x, kx[k][t].x), fminf(mn.y, kx[k][t].y));
          mx = make_float2(fmaxf(mx.x, kx[k][t].x), fmaxf(mx.y, kx[k][t].y));
        }
        kmn_s[wave][2 * cp] = mn.x;
        kmn_s[wave][2 * cp + 1] = mn.y;
        kmx_s[wave][2 * cp] = mx.x;
        kmx_s[wave][2 * cp + 1] = mx.y;
      }
    }
    __syncthreads();
    // key groups of 64 or 128 tokens span several workgroups: their scales and
    // zeros come from key_range_kernel, launched before this kernel
    const int ksh = key_group_shift(a.L.k_group);
    for (int c = tid; c < Dk; c += kPackThreads) {
      if (ksh == 0) {
        float mn = kmn_s[0][c], mx = kmx_s[0][c];
#pragma unroll
        for (int w = 1; w < kPackWaves; ++w) {
          mn = fminf(mn, kmn_s[w][c]);
          mx = fmaxf(mx, kmx_s[w][c]);
        }
        const QParams q = make_qparams(mn, mx, k_levels);
        const int64_t so = (slab * a.g_stride + g) * Dk + c;
        out_store(static_cast<uint16_t*>(a.cache.k_scale) + so, q.s_bits);
        out_store(static_cast<uint16_t*>(a.cache.k_zero) + so, q.z_bits);
        ks_s[c] = q.s;
        kz_s[c] = q.z;
        kr_s[c] = q.r;
      } else {
        const int64_t so = (slab * (a.g_stride >> ksh) + (g >> ksh)) * Dk + c;
        const QParams q = qparams_of(static_cast<const uint16_t*>(a.cache.k_scale)[so],
                                     static_cast<const uint16_t*>(a.cache.k_zero)[so]);
        ks_s[c] = q.s;
        kz_s[c] = q.z;
        kr_s[c] = q.r;
      }
    }
    __syncthreads();
    {
      // key words: row t, word c / (32/KB), channel c at bit (c % (32/KB)) * KB
      // (3 bits: channel c at bit 3c of the row's bit stream);
      // the lane's two channels are adjacent fields of one word
      constexpr int per = 32 / KB;
#pragma unroll
      for (int k = 0; k < kMaxPairBlocks; ++k) {
        const int cp = lane + 64 * k;
        if (2 * cp < Dk) {
          const float s0 = ks_s[2 * cp], z0 = kz_s[2 * cp], r0 = kr_s[2 * cp];
          const float s1 = ks_s[2 * cp + 1], z1 = kz_s[2 * cp + 1], r1 = kr_s[2 * cp + 1];
          const int word = (2 * cp) / per, bit = ((2 * cp) % per) * KB;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t c0 = quant_code(kx[k][t].x, s0, z0, r0, k_levels);
            const uint32_t c1 = quant_code(kx[k][t].y, s1, z1, r1, k_levels);
            const uint32_t f = c0 | (c1 << KB);
            if constexpr (KB == 3) {
              // a bit stream: channel c at bit 3c of the row
              uint32_t* kr = kw_s + (8 * wave + t) * kwords;
              or_code<3>(kr, 6 * cp, c0);
              or_code<3>(kr, 6 * cp + 3, c1);
            } else if constexpr (KB <= 2) {
              atomicOr(&kw_s[(8 * wave + t) * kwords + word], f << bit);
            } else {
              // the lane's two fields fill one byte (4 bits) or two (8 bits) of the
              // word: plain stores, no atomics
              unsigned char* dst = reinterpret_cast<unsigned char*>(kw_s + (8 * wave + t) * kwords + word) + bit / 8;
              if constexpr (KB == 8)
                *reinterpret_cast<uint16_t*>(dst) = uint16_t(f);
              else
                *dst = uint8_t(f);
            }
          }
        }
      }
    }

    // values: per (token, v_group-channel group)
    constexpr float v_levels = float((1 << VB) - 1);
    const int vg = a.L.v_group;
    if (v128) {
      // the thread's 16 channels are one 16-channel tile of the code stream (their
      // codes sit at one bit offset in words 2 * VB apart) and one of the vg / 16
      // adjacent lanes that hold a value group
      float x[16];
      cvt16<DT>(vraw, x);
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int k = 1; k < 16; ++k) {
        mn = fminf(mn, x[k]);
        mx = fmaxf(mx, x[k]);
      }
      mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0xB1, 0xF, 0xF, true)));  // lane ^ 1
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0xB1, 0xF, 0xF, true)));
      if (vg >= 64) {  // lane ^ 2
        mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0x4E, 0xF, 0xF, true)));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x4E, 0xF, 0xF, true)));
      }
      if (vg >= 128) {  // the other quad of the 8 lanes (its lanes already agree)
        mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0x141, 0xF, 0xF, true)));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x141, 0xF, 0xF, true)));
      }
      const QParams q = make_qparams(mn, mx, v_levels);
      const int tiles_per_group = vg >> 4;
      if ((vtile & (tiles_per_group - 1)) == 0) {
        vs_s[vtile / tiles_per_group][vtok] = q.s_bits;
        vz_s[vtile / tiles_per_group][vtok] = q.z_bits;
      }
      const int p0 = value_bit_position(vtok, 16 * vtile, 128, VB);
      const int w0 = p0 >> 5, sh = p0 & 31;
#pragma unroll
      for (int n = 0; n < 16; ++n)
        atomicOr(&vw_s[w0 + n * 2 * VB], quant_code(x[n], q.s, q.z, q.r, v_levels) << sh);
    }
    // other head widths: lanes 16r..16r+15 of a pair block hold 32 channels, the
    // vg / 32 adjacent rows of 16 lanes one value group (all lanes of a group are on)
#pragma unroll
    for (int k = 0; k < kMaxPairBlocks && !v128; ++k) {
      const int cp = lane + 64 * k;
      if (128 * k < Dv) {  // wave-uniform: the pair block reaches into the head
        const bool on = 2 * cp < Dv;
        const int gc = (2 * cp) / vg;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int tok = 8 * wave + t;
          const float2 x = on ? load_pair<DT>(a.V, (slab * a.t_count + rows[t]) * Dv + 2 * cp)
                              : make_float2(0.0f, 0.0f);
          float mn = row16_reduce<false>(fminf(x.x, x.y));
          float mx = row16_reduce<true>(fmaxf(x.x, x.y));
          for (int o = 16; o < vg / 2; o <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, o));
            mx = fmaxf(mx, __shfl_xor(mx, o));
          }
          if (on) {
            const QParams q = make_qparams(mn, mx, v_levels);
            if ((lane & (vg / 2 - 1)) == 0) {
              vs_s[gc][tok] = q.s_bits;
              vz_s[gc][tok] = q.z_bits;
            }
            const uint32_t c0 = quant_code(x.x, q.s, q.z, q.r, v_levels);
            const uint32_t c1 = quant_code(x.y, q.s, q.z, q.r, v_levels);
            const int p0 = value_bit_position(tok, 2 * cp, Dv, VB), p1 = value_bit_position(tok, 2 * cp + 1, Dv, VB);
            or_code<VB>(vw_s, p0, c0);
            or_code<VB>(vw_s, p1, c1);
          }
        }
      }
    }
    __syncthreads();

    // contiguous stores of the group's key words, value stream and value scale / zero
    // (streaming stores, as every output of this kernel: see out_store)
    uint32_t* kdst = static_cast<uint32_t*>(a.cache.k_codes) + ((slab * a.g_stride + g) * KVQ_GROUP) * kwords;
    for (int i = tid; i < KVQ_GROUP * kwords; i += kPackThreads) out_store(kdst + i, kw_s[i]);
    uint32_t* vdst = static_cast<uint32_t*>(a.cache.v_codes) + (slab * a.g_stride + g) * vwords;
    for (int i = tid; i < vwords; i += kPackThreads) out_store(vdst + i, vw_s[i]);
    const int ngv = Dv / vg;
    const int64_t vso = (slab * a.g_stride + g) * ngv * KVQ_GROUP;
    for (int i = tid; i < ngv * KVQ_GROUP; i += kPackThreads) {
      out_store(static_cast<uint16_t*>(a.cache.v_scale) + vso + i, vs_s[i / KVQ_GROUP][i % KVQ_GROUP]);
      out_store(static_cast<uint16_t*>(a.cache.v_zero) + vso + i, vz_s[i / KVQ_GROUP][i % KVQ_GROUP]);
    }
  } else {
    // ------------------------------------------------ retained rows -> fp16
    const int sub = tid / (kPackThreads / kRetRowsPerBlock);
    const int lt = tid % (kPackThreads / kRetRowsPerBlock);
    const int64_t j = (int64_t(blockIdx.x) - a.n_groups_chunk) * kRetRowsPerBlock + sub;
    if (j >= a.n_ret_chunk) return;
    const int64_t r = a.r_begin + j;                           // rank among all retained rows
    const int64_t row = retained_position(rr, r) - a.t_begin;  // row in the chunk
    uint16_t* kd = static_cast<uint16_t*>(a.cache.k_fp16) + (slab * a.r_stride + r) * Dk;
    uint16_t* vd = static_cast<uint16_t*>(a.cache.v_fp16) + (slab * a.r_stride + r) * Dv;
    static_assert(kPackThreads / kRetRowsPerBlock == 64 && KVQ_MAX_HEAD_DIM <= 256, "one wave per retained row");
    if (a.L.flags & KVQ_KEY_ROTATION) {
      // the wave holds the row as x[j] = channel lane + 64j: butterflies h = 1 .. 32
      // with lane ^ h, then 64 and 128 across j
      float x[4];
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        const int c = lt + 64 * j2;
        x[j2] = c < Dk ? load_elem<DT>(a.K, (slab * a.t_count + row) * Dk + c) : 0.0f;
      }
      for (int hl = 1; hl < 64 && hl < Dk; hl <<= 1) {
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) x[j2] = butterfly(x[j2], __shfl_xor(x[j2], hl), (lt & hl) != 0);
      }
      if (Dk > 64) {
        const float u0 = x[0], u1 = x[1], u2 = x[2], u3 = x[3];
        x[0] = u0 + u1; x[1] = u0 - u1; x[2] = u2 + u3; x[3] = u2 - u3;
      }
      if (Dk > 128) {
        const float u0 = x[0], u1 = x[1], u2 = x[2], u3 = x[3];
        x[0] = u0 + u2; x[1] = u1 + u3; x[2] = u0 - u2; x[3] = u1 - u3;
      }
      const float sc = rotation_scale(31 - __builtin_clz(unsigned(Dk)));
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        const int c = lt + 64 * j2;
        if (c < Dk) out_store(kd + c, f16_bits_rne(rotation_scaled(x[j2], sc)));
      }
    } else {
      for (int c = lt; c < Dk; c += kPackThreads / kRetRowsPerBlock)
        out_store(kd + c, f16_bits_rne(load_elem<DT>(a.K, (slab * a.t_count + row) * Dk + c)));
    }
    for (int c = lt; c < Dv; c += kPackThreads / kRetRowsPerBlock)
      out_store(vd + c, f16_bits_rne(load_elem<DT>(a.V, (slab * a.t_count + row) * Dv + c)));
  }
}

// Key rotation of a 128-wide row held by 16 consecutive lanes, lane c owning
// channels 8c .. 8c+7: butterflies 1, 2, 4 in registers, 8 .. 64 with lane c ^ h/8.
__device__ __forceinline__ void rotate_row128(float (&x)[8], int c) {
  butterflies8(x);
#pragma unroll
  for (int hl = 1; hl < 16; hl <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = butterfly(x[k], __shfl_xor(x[k], hl), (c & hl) != 0);
  }
  const float sc = rotation_scale(7);
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = rotation_scaled(x[k], sc);
}

// Pack kernel for the common shape: Dk = Dv = 128, 32-token key groups, 2/4/8-bit
// codes, 16-bit inputs.  Same contract and outputs as pack_kernel; arranged so
// that every load is a 16-byte row segment and the codes leave in whole words.
// Workgroup = one key group; wave w holds tokens 8w..8w+7 (one octet of the value
// code layout), lane (p = lane / 16, c = lane % 16) the channels 8c..8c+7 of the
// token pair (8w + p, 8w + p + 4):
//   keys    per-channel min / max: lane partials through LDS (16 per channel),
//           reduced by one thread per channel, which also forms the scale and zero;
//           each lane's 8 codes of a row are whole key-code bits of one word (4- and
//           8-bit: 1 or 2 words; 2-bit: half a word, joined with the next lane), stored
//           straight to the cache;
//   values  per (token, v_group channels) min / max over the 8 lanes' quads (DPP),
//           scale and zero formed by one lane per token of a quad; the lane's codes
//           of tile t = c / 2, columns 8 (c % 2) + k, make 8 partial words, one for each
//           of 8 words of its wave's octet; each goes to its own LDS slot (word, t % TPW),
//           so every slot is written once with a plain store, and each lane then ORs
//           the TPW slots of the words it stores.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int DT, int KB, int VB>
__global__ __launch_bounds__(kPackThreads) void pack128_kernel(const PackArgs a) {
  static_assert(DT != KVQ_F32 && (KB == 2 || KB == 4 || KB == 8) && (VB == 2 || VB == 4 || VB == 8), "shape");
  constexpr int D = 128, kWords = D * KB / 32, vWords = D * VB;
  constexpr int kChunkWords = VB / 2;             // words of a (octet, column, pair) field
  constexpr int kTilesPerWord = 16 / VB;
  __shared__ int32_t row_s[KVQ_GROUP];
  // the key partials (lane partials: (wave, pair) x channel) are dead after the
  // second barrier, when the value slots (per wave: (word, tile slot) partial words)
  // come into use: they share the memory
  __shared__ __align__(16) float4 part_s[2 * 16 * (D / 4)];
  float4 (*kmn_s)[D / 4] = reinterpret_cast<float4 (*)[D / 4]>(part_s);
  float4 (*kmx_s)[D / 4] = reinterpret_cast<float4 (*)[D / 4]>(part_s + 16 * (D / 4));
  static_assert(sizeof(float4) * 2 * 16 * (D / 4) >= sizeof(uint32_t) * kPackWaves * 64 * 8, "value slots");
  __shared__ float4 ks_s[D / 4], kz_s[D / 4], kr_s[D / 4], knzr_s[D / 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  const RetentionRule rr{a.L.T, a.L.n_recent, a.L.log_window};

  if (int64_t(blockIdx.x) >= a.n_groups_chunk) {
    // retained rows -> fp16: kRetRows128 rows per workgroup, 16 threads per row, 8
    // channels (one 16-byte load of K and of V) per thread
    for (int i = tid; i < kRetRows128 * 16; i += kPackThreads) {
      const int64_t j = (int64_t(blockIdx.x) - a.n_groups_chunk) * kRetRows128 + i / 16;
      if (j >= a.n_ret_chunk) break;
      const int c8 = 8 * (i % 16);
      const int64_t r = a.r_begin + j;
      const int64_t e = (slab * a.t_count + (retained_position(rr, r) - a.t_begin)) * D + c8;
      const uint4 kv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.K) + e);
      const uint4 vv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.V) + e);
      const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
      u32x4_t ko, vo;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (DT == KVQ_BF16) {
          ko[k] = uint32_t(f16_bits_rne(__uint_as_float(kw[k] << 16))) |
                  (uint32_t(f16_bits_rne(__uint_as_float(kw[k] & 0xFFFF0000u))) << 16);
          vo[k] = uint32_t(f16_bits_rne(__uint_as_float(vw[k] << 16))) |
                  (uint32_t(f16_bits_rne(__uint_as_float(vw[k] & 0xFFFF0000u))) << 16);
        } else {  // fp16 rows are stored as they are
          ko[k] = kw[k];
          vo[k] = vw[k];
        }
      }
      if (a.L.flags & KVQ_KEY_ROTATION) {
        // the row's 16 threads are 16 consecutive lanes (i % 16 == lane % 16)
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (DT == KVQ_BF16) {
            x[2 * k] = __uint_as_float(kw[k] << 16);
            x[2 * k + 1] = __uint_as_float(kw[k] & 0xFFFF0000u);
          } else {
            x[2 * k] = __half2float(__ushort_as_half(uint16_t(kw[k] & 0xFFFFu)));
            x[2 * k + 1] = __half2float(__ushort_as_half(uint16_t(kw[k] >> 16)));
          }
        }
        rotate_row128(x, i % 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) ko[k] = uint32_t(f16_bits_rne(x[2 * k])) | (uint32_t(f16_bits_rne(x[2 * k + 1])) << 16);
      }
      out_store(reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.cache.k_fp16) + (slab * a.r_stride + r) * D + c8), ko);
      out_store(reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.cache.v_fp16) + (slab * a.r_stride + r) * D + c8), vo);
    }
    return;
  }

  const int64_t g = a.g_begin + blockIdx.x;
  const bool plain = quantized_before(rr, (g + 1) * KVQ_GROUP) == (g + 1) * KVQ_GROUP;
  if (!plain) {
    if (tid < KVQ_GROUP) row_s[tid] = int32_t(quantized_position(rr, g * KVQ_GROUP + tid) - a.t_begin);
    __syncthreads();
  }
  const int p = lane >> 4, c = lane & 15;
  const int tok[2] = {8 * wave + p, 8 * wave + p + 4};
  // wave-uniform 64-bit bases, 32-bit lane offsets (a slab's chunk is < 2^31 bytes)
  const uint16_t* Kb = static_cast<const uint16_t*>(a.K) + slab * a.t_count * D;
  const uint16_t* Vb = static_cast<const uint16_t*>(a.V) + slab * a.t_count * D;
  const int32_t row0 = int32_t(g * KVQ_GROUP - a.t_begin);  // chunk row of token 0 of a plain group
  Raw16<DT> kraw[2], vraw[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t row = uint32_t(plain ? row0 + tok[j] : row_s[tok[j]]);
    const uint32_t e = row * D + 8 * c;
    const uint4 kv = *reinterpret_cast<const uint4*>(Kb + e);
    const uint4 vv = *reinterpret_cast<const uint4*>(Vb + e);
    kraw[j].w[0] = kv.x; kraw[j].w[1] = kv.y; kraw[j].w[2] = kv.z; kraw[j].w[3] = kv.w;
    vraw[j].w[0] = vv.x; vraw[j].w[1] = vv.y; vraw[j].w[2] = vv.z; vraw[j].w[3] = vv.w;
  }
  // 16-bit words -> floats (values stay raw until the value phase)
  auto widen = [](const Raw16<DT>& r, float (&x)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (DT == KVQ_BF16) {
        x[2 * k] = __uint_as_float(r.w[k] << 16);
        x[2 * k + 1] = __uint_as_float(r.w[k] & 0xFFFF0000u);
      } else {
        x[2 * k] = __half2float(__ushort_as_half(uint16_t(r.w[k] & 0xFFFFu)));
        x[2 * k + 1] = __half2float(__ushort_as_half(uint16_t(r.w[k] >> 16)));
      }
    }
  };
  float kx[2][8];
  widen(kraw[0], kx[0]);
  widen(kraw[1], kx[1]);
  if (a.L.flags & KVQ_KEY_ROTATION) {  // wave-uniform
    rotate_row128(kx[0], c);
    rotate_row128(kx[1], c);
  }

  // ---------------------------------------------------------------- keys
  {
    float mn[8], mx[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mn[k] = fminf(kx[0][k], kx[1][k]);
      mx[k] = fmaxf(kx[0][k], kx[1][k]);
    }
    const int pr = wave * 4 + p;
    kmn_s[pr][2 * c] = make_float4(mn[0], mn[1], mn[2], mn[3]);
    kmn_s[pr][2 * c + 1] = make_float4(mn[4], mn[5], mn[6], mn[7]);
    kmx_s[pr][2 * c] = make_float4(mx[0], mx[1], mx[2], mx[3]);
    kmx_s[pr][2 * c + 1] = make_float4(mx[4], mx[5], mx[6], mx[7]);
  }
  __syncthreads();
  constexpr float k_levels = float((1 << KB) - 1);
  if (tid < D) {
    const float* mnp = reinterpret_cast<const float*>(kmn_s);
    const float* mxp = reinterpret_cast<const float*>(kmx_s);
    float mn = mnp[tid], mx = mxp[tid];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      mn = fminf(mn, mnp[r * D + tid]);
      mx = fmaxf(mx, mxp[r * D + tid]);
    }
    const QParams q = make_qparams(mn, mx, k_levels);
    const int64_t so = (slab * a.g_stride + g) * D;
    out_store(static_cast<uint16_t*>(a.cache.k_scale) + so + uint32_t(tid), q.s_bits);
    out_store(static_cast<uint16_t*>(a.cache.k_zero) + so + uint32_t(tid), q.z_bits);
    reinterpret_cast<float*>(ks_s)[tid] = q.s;
    reinterpret_cast<float*>(kz_s)[tid] = q.z;
    reinterpret_cast<float*>(kr_s)[tid] = q.r;
    reinterpret_cast<float*>(knzr_s)[tid] = -q.z * q.r;
  }
  __syncthreads();
  {
    float kr[8], knzr[8];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      const float4 r4 = kr_s[2 * c + hq], n4 = knzr_s[2 * c + hq];
      kr[4 * hq] = r4.x; kr[4 * hq + 1] = r4.y; kr[4 * hq + 2] = r4.z; kr[4 * hq + 3] = r4.w;
      knzr[4 * hq] = n4.x; knzr[4 * hq + 1] = n4.y; knzr[4 * hq + 2] = n4.z; knzr[4 * hq + 3] = n4.w;
    }
    float nmax = 0.0f, rmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      nmax = fmaxf(nmax, fabsf(knzr[k]));
      rmax = fmaxf(rmax, kr[k]);
    }
    const float klim = fma_quant_limit(nmax);
    const bool kclamp = !__all(clamp_free(nmax, rmax));
    const float* ksf = reinterpret_cast<const float*>(ks_s) + 8 * c;
    const float* kzf = reinterpret_cast<const float*>(kz_s) + 8 * c;
    uint32_t* kdst = static_cast<uint32_t*>(a.cache.k_codes) + ((slab * a.g_stride + g) * KVQ_GROUP) * kWords;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t lo = 0, hi = 0;  // channels 8c .. 8c+7 at bits (k * KB) of a 64-bit field
      float q[8];
      quant_levels_fma<8>(kx[j], kr, knzr, klim, k_levels, kclamp, q,
                          [&](int k) { return (kx[j][k] - kzf[k]) / ksf[k]; });
      if constexpr (KB == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo = put_byte(q[k], k, lo);
          hi = put_byte(q[4 + k], k, hi);
        }
      } else if constexpr (KB == 4) {
        // even channels in the low nibbles of the bytes, odd ones in the high
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ev = put_byte(q[2 * k], k, ev);
          od = put_byte(q[2 * k + 1], k, od);
        }
        lo = ev | (od << 4);
      } else {
        // channel k at bits 2k: byte k / 4, bit pair k % 4
        uint32_t f[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k) f[k & 3] = put_byte(q[k], k >> 2, f[k & 3]);
        lo = f[0] | (f[1] << 2) | (f[2] << 4) | (f[3] << 6);
      }
      uint32_t* rowp = kdst + uint32_t(tok[j] * kWords);
      if constexpr (KB == 8) {
        out_store(reinterpret_cast<u32x2_t*>(rowp) + c, u32x2_t{lo, hi});
      } else if constexpr (KB == 4) {
        out_store(rowp + c, lo);
      } else {
        // 16 bits per lane: lanes 2m, 2m + 1 fill word m
        const uint32_t nb = uint32_t(__builtin_amdgcn_mov_dpp(int(lo), 0xB1, 0xF, 0xF, true));  // lane ^ 1
        if ((c & 1) == 0) out_store(rowp + (c >> 1), lo | (nb << 16));
      }
    }
  }

  // -------------------------------------------------------------- values
  constexpr float v_levels = float((1 << VB) - 1);
  // channels and lanes per value group (v_group is 32, 64 or 128: shifts, no divides)
  const int vsh = a.L.v_group == 128 ? 2 : (a.L.v_group == 64 ? 1 : 0);
  const int lpg = 4 << vsh;
  uint32_t* slots = reinterpret_cast<uint32_t*>(part_s) + wave * (64 * 8);  // this wave's alone, in issue order
  float vx[2][8];
  widen(vraw[0], vx[0]);
  widen(vraw[1], vx[1]);
  float vmn[2], vmx[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float mn = vx[j][0], mx = vx[j][0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      mn = fminf(mn, vx[j][k]);
      mx = fmaxf(mx, vx[j][k]);
    }
    mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0xB1, 0xF, 0xF, true)));  // lane ^ 1
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0xB1, 0xF, 0xF, true)));
    mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0x4E, 0xF, 0xF, true)));  // lane ^ 2
    mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x4E, 0xF, 0xF, true)));
    if (lpg >= 8) {
      mn = fminf(mn, __shfl_xor(mn, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 4));
    }
    if (lpg >= 16) {
      mn = fminf(mn, __shfl_xor(mn, 8));
      mx = fmaxf(mx, __shfl_xor(mx, 8));
    }
    vmn[j] = mn;
    vmx[j] = mx;
  }
  // lane c forms the parameters of row c & 1; the other row's come from lane c ^ 1
  const int jm = c & 1;
  const QParams qm = make_qparams(jm ? vmn[1] : vmn[0], jm ? vmx[1] : vmx[0], v_levels);
  const float os = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(qm.s), 0xB1, 0xF, 0xF, true));
  const float oz = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(qm.z), 0xB1, 0xF, 0xF, true));
  const float orr = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(qm.r), 0xB1, 0xF, 0xF, true));
  const float vs[2] = {jm ? os : qm.s, jm ? qm.s : os};
  const float vz[2] = {jm ? oz : qm.z, jm ? qm.z : oz};
  const float vr[2] = {jm ? orr : qm.r, jm ? qm.r : orr};
  if ((c & (lpg - 1)) < 2) {
    // one lane per (token, value group) stores its scale and zero
    const int ngv = D >> (5 + vsh), gc = (8 * c) >> (5 + vsh);
    const int64_t vso = (slab * a.g_stride + g) * ngv * KVQ_GROUP;
    const uint32_t vo = uint32_t(gc * KVQ_GROUP + tok[jm]);
    out_store(static_cast<uint16_t*>(a.cache.v_scale) + vso + vo, qm.s_bits);
    out_store(static_cast<uint16_t*>(a.cache.v_zero) + vso + vo, qm.z_bits);
  }
  {
    // the lane's codes: tile t = c / 2, columns 8 (c % 2) + k, tokens pair (p, p + 4)
    const int t = c >> 1, hc = c & 1;
    const int chunk = t / kTilesPerWord, slot = t % kTilesPerWord;
    uint32_t part[8];
    float c0[8], c1[8];
    {
      float r8[8], n8[8];
      const float n0 = -vz[0] * vr[0], n1 = -vz[1] * vr[1];
      const bool vclamp = !__all(clamp_free(fmaxf(fabsf(n0), fabsf(n1)), fmaxf(vr[0], vr[1])));
#pragma unroll
      for (int k = 0; k < 8; ++k) { r8[k] = vr[0]; n8[k] = n0; }
      quant_levels_fma<8>(vx[0], r8, n8, fma_quant_limit(fabsf(n0)), v_levels, vclamp, c0,
                          [&](int k) { return (vx[0][k] - vz[0]) / vs[0]; });
#pragma unroll
      for (int k = 0; k < 8; ++k) { r8[k] = vr[1]; n8[k] = n1; }
      quant_levels_fma<8>(vx[1], r8, n8, fma_quant_limit(fabsf(n1)), v_levels, vclamp, c1,
                          [&](int k) { return (vx[1][k] - vz[1]) / vs[1]; });
    }
    // token p's code at bit slot * VB, token p + 4's 16 bits higher
#pragma unroll
    for (int k = 0; k < 8; ++k) part[k] = put_byte(c1[k], 2, put_byte(c0[k], 0, 0u)) << (slot * VB);
    // column n = 8 hc + k: word (field (n * 4 + p) of the octet, chunk), slot t % TPW;
    // (word, slot) = 8 (n * 4 + p) + t since a field's chunks hold 8 tiles' slots
#pragma unroll
    for (int k = 0; k < 8; ++k) slots[8 * ((8 * hc + k) * 4 + p) + t] = part[k];
    (void)chunk;
  }
  // the octet's words, contiguous in the group's stream: field (16 wave + n) * 4 + p
  // is words kChunkWords * ((n * 4 + p)) .. of the wave's block; lane l stores words
  // kChunkWords * l .. kChunkWords * l + kChunkWords - 1, each the OR of its TPW slots
  uint32_t wv[kChunkWords];
#pragma unroll
  for (int i = 0; i < kChunkWords; ++i) {
    const int word = kChunkWords * lane + i;
    uint32_t v = 0;
#pragma unroll
    for (int m = 0; m < kTilesPerWord; ++m) v |= slots[word * kTilesPerWord + m];
    wv[i] = v;
  }
  uint32_t* vdst = static_cast<uint32_t*>(a.cache.v_codes) + (slab * a.g_stride + g) * vWords + wave * (32 * VB);
  if constexpr (kChunkWords == 1) {
    out_store(vdst + uint32_t(lane), wv[0]);
  } else if constexpr (kChunkWords == 2) {
    out_store(reinterpret_cast<u32x2_t*>(vdst) + uint32_t(lane), u32x2_t{wv[0], wv[1]});
  } else {
    out_store(reinterpret_cast<u32x4_t*>(vdst) + uint32_t(lane), u32x4_t{wv[0], wv[1], wv[2], wv[3]});
  }
}

// Key groups of k_group = 64 or 128 tokens: per-channel min / max over the key
// group's tokens, then its scale and zero (make_qparams, as for 32-token groups).
// One workgroup per (key group of the chunk, kv head, batch row); thread (channel
// c, slice sl) takes tokens sl, sl + nsl, ...; the slices meet in LDS.
template <int DT>
__global__ __launch_bounds__(kPackThreads) void key_range_kernel(const PackArgs a) {
  __shared__ float mn_s[kPackThreads], mx_s[kPackThreads];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int Dk = a.L.Dk, kg = a.L.k_group, ksh = key_group_shift(kg);
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  const RetentionRule rr{a.L.T, a.L.n_recent, a.L.log_window};
  const int64_t kj = (a.g_begin >> ksh) + blockIdx.x;  // key group in the slab
  const int64_t q0 = kj * kg;                          // its first compacted token
  const bool plain = quantized_before(rr, q0 + kg) == q0 + kg;
  const int nsl = kPackThreads / Dk;
  const int c = tid % Dk, sl = tid / Dk;
  float mn = INFINITY, mx = -INFINITY;
  if (a.L.flags & KVQ_KEY_ROTATION) {
    // rotated keys: Dk is a power of two, so the workgroup is nsl whole rows and
    // every thread takes part; each pass rotates nsl rows through LDS, butterflies
    // in increasing h (partner channel c ^ h of the same row)
    for (int t0 = 0; t0 < kg; t0 += nsl) {
      const int t = t0 + sl;
      const int64_t row = (plain ? q0 + t : quantized_position(rr, q0 + t)) - a.t_begin;
      float x = load_elem<DT>(a.K, (slab * a.t_count + row) * Dk + c);
      for (int hh = 1; hh < Dk; hh <<= 1) {
        mn_s[tid] = x;
        __syncthreads();
        const float partner = mn_s[tid ^ hh];
        __syncthreads();
        x = butterfly(x, partner, (c & hh) != 0);
      }
      x = rotation_scaled(x, rotation_scale(31 - __builtin_clz(unsigned(Dk))));
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
  } else if (sl < nsl) {
    for (int t = sl; t < kg; t += nsl) {
      const int64_t row = (plain ? q0 + t : quantized_position(rr, q0 + t)) - a.t_begin;
      const float x = load_elem<DT>(a.K, (slab * a.t_count + row) * Dk + c);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
  }
  mn_s[tid] = mn;
  mx_s[tid] = mx;
  __syncthreads();
  if (tid < Dk) {
    for (int i = 1; i < nsl; ++i) {
      mn = fminf(mn, mn_s[i * Dk + tid]);
      mx = fmaxf(mx, mx_s[i * Dk + tid]);
    }
    const QParams q = make_qparams(mn, mx, float((1 << a.L.k_bits) - 1));
    const int64_t so = (slab * (a.g_stride >> ksh) + kj) * Dk + tid;
    out_store(static_cast<uint16_t*>(a.cache.k_scale) + so, q.s_bits);
    out_store(static_cast<uint16_t*>(a.cache.k_zero) + so, q.z_bits);
  }
}

template <int DT>
hipError_t launch_dt(const PackArgs& a, dim3 grid, hipStream_t stream) {
  const int ksh = key_group_shift(a.L.k_group);
  if (ksh > 0 && a.n_groups_chunk > 0) {
    const dim3 kgrid(unsigned(a.n_groups_chunk >> ksh), unsigned(a.L.Hkv), unsigned(a.L.B));
    hipLaunchKernelGGL((key_range_kernel<DT>), kgrid, dim3(kPackThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int kb = a.L.k_bits, vb = a.L.v_bits;
  if constexpr (DT != KVQ_F32) {
    if (a.L.Dk == 128 && a.L.Dv == 128 && a.L.k_group == 32) {
      const dim3 g128(unsigned(a.n_groups_chunk + (a.n_ret_chunk + kRetRows128 - 1) / kRetRows128), grid.y, grid.z);
#define KVQ_PACK128_CASE(K_, V_)                                                                    \
      if (kb == K_ && vb == V_) {                                                                   \
        hipLaunchKernelGGL((pack128_kernel<DT, K_, V_>), g128, dim3(kPackThreads), 0, stream, a);  \
        return hipGetLastError();                                                                   \
      }
      KVQ_PACK128_CASE(2, 2) KVQ_PACK128_CASE(2, 4) KVQ_PACK128_CASE(2, 8)
      KVQ_PACK128_CASE(4, 2) KVQ_PACK128_CASE(4, 4) KVQ_PACK128_CASE(4, 8)
      KVQ_PACK128_CASE(8, 2) KVQ_PACK128_CASE(8, 4) KVQ_PACK128_CASE(8, 8)
#undef KVQ_PACK128_CASE
    }
  }
#define KVQ_PACK_CASE(K_, V_)                                                                     \
  if (kb == K_ && vb == V_) {                                                                     \
    hipLaunchKernelGGL((pack_kernel<DT, K_, V_>), grid, dim3(kPackThreads), 0, stream, a);       \
    return hipGetLastError();                                                                     \
  }
  KVQ_PACK_CASE(1, 1) KVQ_PACK_CASE(1, 2) KVQ_PACK_CASE(1, 4) KVQ_PACK_CASE(1, 8)
  KVQ_PACK_CASE(2, 1) KVQ_PACK_CASE(2, 2) KVQ_PACK_CASE(2, 4) KVQ_PACK_CASE(2, 8)
  KVQ_PACK_CASE(4, 1) KVQ_PACK_CASE(4, 2) KVQ_PACK_CASE(4, 4) KVQ_PACK_CASE(4, 8)
  KVQ_PACK_CASE(8, 1) KVQ_PACK_CASE(8, 2) KVQ_PACK_CASE(8, 4) KVQ_PACK_CASE(8, 8)
  KVQ_PACK_CASE(3, 1) KVQ_PACK_CASE(3, 2) KVQ_PACK_CASE(3, 3) KVQ_PACK_CASE(3, 4) KVQ_PACK_CASE(3, 8)
  KVQ_PACK_CASE(1, 3) KVQ_PACK_CASE(2, 3) KVQ_PACK_CASE(4, 3) KVQ_PACK_CASE(8, 3)
#undef KVQ_PACK_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
  const int64_t nblk = a.n_groups_chunk + (a.n_ret_chunk + kRetRowsPerBlock - 1) / kRetRowsPerBlock;
  if (nblk == 0) return hipSuccess;
  const dim3 grid(unsigned(nblk), unsigned(a.L.Hkv), unsigned(a.L.B));
  switch (a.dtype) {
    case KVQ_F32: return launch_dt<KVQ_F32>(a, grid, stream);
    case KVQ_F16: return launch_dt<KVQ_F16>(a, grid, stream);
    case KVQ_BF16: return launch_dt<KVQ_BF16>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// ----------------------------------------------------- HeadQ side code (write path)
// Thread (token t = tid / 16, coefficient k = tid % 16) of the workgroup of code
// group g: y_k = sum_c (k_c - k_hat_c) U[c][k] in float64, channels in ascending
// order with no fused multiply-add, rounded once to float32; then the token's r
// coefficients are one quantizer group (the library's min/max contract).
namespace {
template <int DT>
__device__ __forceinline__ float load_one(const void* p, int64_t i) {
  if constexpr (DT == KVQ_F32) return static_cast<const float*>(p)[i];
  else if constexpr (DT == KVQ_F16) return __half2float(static_cast<const __half*>(p)[i]);
  else return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
}

template <int DT>
__global__ __launch_bounds__(KVQ_GROUP * kMaxSideRank) void side_pack_kernel(const SideArgs a) {
  __shared__ float ys[KVQ_GROUP][kMaxSideRank];
  const int g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = int(threadIdx.x) / kMaxSideRank, k = int(threadIdx.x) % kMaxSideRank;
  const int Dk = a.L.Dk, kb = a.L.k_bits, R = a.rank;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  const int64_t Tq = a.L.Tq;
  const int64_t j = int64_t(g) * KVQ_GROUP + t;  // compacted token
  const RetentionRule rule{a.L.T, a.L.n_recent, a.L.log_window};
  const int ksh = key_group_shift(a.L.k_group);
  if (k < R) {
    const int64_t pos = quantized_position(rule, j);
    const uint32_t* row = static_cast<const uint32_t*>(a.cache.k_codes) + (slab * Tq + j) * (Dk * kb / 32);
    const int64_t kgi = slab * (Tq / a.L.k_group) + (g >> ksh);
    const uint16_t* ks = static_cast<const uint16_t*>(a.cache.k_scale) + kgi * Dk;
    const uint16_t* kz = static_cast<const uint16_t*>(a.cache.k_zero) + kgi * Dk;
    const int64_t krow = (slab * a.L.T + pos) * Dk;
    double y = 0.0;
    for (int c = 0; c < Dk; ++c) {
      // k_hat = code * s + z is exact in float64
      const double khat = double(stream_code(row, c * kb, kb)) * double(f16_bits_to_f32(ks[c])) +
                          double(f16_bits_to_f32(kz[c]));
      const double e = __dsub_rn(double(load_one<DT>(a.K, krow + c)), khat);
      y = __dadd_rn(y, __dmul_rn(e, double(a.U[(int64_t(h) * Dk + c) * R + k])));
    }
    ys[t][k] = float(y);
  }
  __syncthreads();
  if (k < R) {
    float mn = ys[t][0], mx = ys[t][0];
    for (int i = 1; i < R; ++i) {
      mn = fminf(mn, ys[t][i]);
      mx = fmaxf(mx, ys[t][i]);
    }
    const float levels = float((1 << a.bits) - 1);
    const QParams q = make_qparams(mn, mx, levels);
    a.codes[(slab * Tq + j) * R + k] = uint8_t(quant_code(ys[t][k], q.s, q.z, q.r, levels));
    if (k == 0) {
      a.scale[slab * Tq + j] = q.s_bits;
      a.zero[slab * Tq + j] = q.z_bits;
    }
  }
}
}  // namespace

hipError_t launch_side_pack(const SideArgs& a, hipStream_t stream) {
  const dim3 grid(unsigned(a.L.n_groups), unsigned(a.L.Hkv), unsigned(a.L.B)), block(KVQ_GROUP * kMaxSideRank);
  switch (a.dtype) {
    case KVQ_F32: hipLaunchKernelGGL(side_pack_kernel<KVQ_F32>, grid, block, 0, stream, a); break;
    case KVQ_F16: hipLaunchKernelGGL(side_pack_kernel<KVQ_F16>, grid, block, 0, stream, a); break;
    case KVQ_BF16: hipLaunchKernelGGL(side_pack_kernel<KVQ_BF16>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
