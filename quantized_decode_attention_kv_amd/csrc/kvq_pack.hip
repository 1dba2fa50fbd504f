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
// One launch per call.  Workgroups [0, n_groups_chunk) each own one key group of
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
// replaced by a multiply with fl(1/s): the two quotients differ by at most
// 3 * 2^-24 * |t| (< 5e-5 while |t| <= 256; a larger |t| clamps the same way), so
// rint gives the same integer unless the quotient lies within 2^-12 of a
// half-integer; such elements (about one in two thousand) take the exact division.
// Scale and zero use the exact division, with contraction off, as the contract
// spells out.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.hpp"
#include "kvq_retention.hpp"
#include "kvq_vlayout.hpp"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackWaves = kPackThreads / 64;
constexpr int kRetRowsPerBlock = 4;
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

// s = fp16(fp32(mx - mn) / (2^bits - 1)), z = fp16(mn); zeros stored as +0.
__device__ __forceinline__ QParams make_qparams(float mn, float mx, float levels) {
  const float range = mx - mn;
  const float s32 = range / levels;
  uint16_t sb = f16_bits_rne(s32);
  uint16_t zb = f16_bits_rne(mn);
  if ((sb & 0x7fffu) == 0) sb = 0;
  if ((zb & 0x7fffu) == 0) zb = 0;
  QParams q;
  q.s_bits = sb;
  q.z_bits = zb;
  q.s = f16_bits_to_f32(sb);
  q.z = f16_bits_to_f32(zb);
  q.r = q.s == 0.0f ? 0.0f : 1.0f / q.s;
  return q;
}

// the same parameters from stored fp16 bits (key groups longer than 32 tokens)
__device__ __forceinline__ QParams qparams_of(uint16_t sb, uint16_t zb) {
  QParams q;
  q.s_bits = sb;
  q.z_bits = zb;
  q.s = f16_bits_to_f32(sb);
  q.z = f16_bits_to_f32(zb);
  q.r = q.s == 0.0f ? 0.0f : 1.0f / q.s;
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

// min / max over the 16 lanes of a DPP row (every lane gets the result)
template <bool MAX>
__device__ __forceinline__ float row16_reduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));   // quad_perm 1,0,3,2
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));  // row_mirror
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
      if (2 * cp < Dk) {
#pragma unroll
        for (int t = 0; t < 8; ++t) kx[k][t] = load_pair<DT>(a.K, (slab * a.t_count + rows[t]) * Dk + 2 * cp);
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
      mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0xB1, 0xF, 0xF, false)));  // lane ^ 1
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0xB1, 0xF, 0xF, false)));
      if (vg >= 64) {  // lane ^ 2
        mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0x4E, 0xF, 0xF, false)));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x4E, 0xF, 0xF, false)));
      }
      if (vg >= 128) {  // the other quad of the 8 lanes (its lanes already agree)
        mn = fminf(mn, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mn), 0x141, 0xF, 0xF, false)));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x141, 0xF, 0xF, false)));
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
    for (int c = lt; c < Dk; c += kPackThreads / kRetRowsPerBlock)
      out_store(kd + c, f16_bits_rne(load_elem<DT>(a.K, (slab * a.t_count + row) * Dk + c)));
    for (int c = lt; c < Dv; c += kPackThreads / kRetRowsPerBlock)
      out_store(vd + c, f16_bits_rne(load_elem<DT>(a.V, (slab * a.t_count + row) * Dv + c)));
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
  if (sl < nsl) {
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
