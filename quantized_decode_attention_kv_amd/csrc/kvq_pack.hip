// kv_quant_pack kernel for gfx950.
//
// Group-wise asymmetric min/max quantization with fp16 scale/zero: keys per
// channel over 32 consecutive quantized tokens ("LogQuant: Log-Distributed 2-Bit
// Quantization of KV Cache", section 5, per-channel keys; group 32 from "Quantize
// What Counts: More for Keys, Less for Values", results), values per token over 32
// channels, separate key / value bit widths (Quantize What Counts, methodology).
// Retained positions (LogQuant section 2) are copied to fp16 rows.
//
// One launch per call.  Blocks [0, n_groups_chunk) each own one key group of one
// (batch, kv-head) slab: its 32 token rows of K and V are read once, coalesced
// along channels; per-channel key min/max is a register reduction over the 32
// tokens a thread holds, per-token value min/max is a 32-lane shuffle reduction;
// codes are staged in LDS and packed into 32-bit words by consecutive threads, so
// every global store is a coalesced run.  The remaining
// blocks copy the chunk's retained rows to fp16.
//
// The quantize arithmetic is kept in the exact float32 order of the contract in
// kvq.h (correctly rounded division, no contraction) so codes and fp16 bits are
// reproducible bit for bit.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.hpp"
#include "kvq_retention.hpp"
#include "kvq_vlayout.hpp"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kPackThreads = 256;
constexpr int kRetRowsPerBlock = 4;

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

__device__ __forceinline__ uint16_t f16_bits_rne(float x) {
  return __half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

struct QParams {
  float s, z;
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
  return q;
}

__device__ __forceinline__ uint32_t quant_code(float x, const QParams& q, float levels) {
  if (q.s == 0.0f) return 0u;
  const float t = (x - q.z) / q.s;
  float r = __builtin_rintf(t);
  r = fminf(fmaxf(r, 0.0f), levels);
  return uint32_t(r);
}

__device__ __forceinline__ float group32_min(float v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 32));
  return v;
}
__device__ __forceinline__ float group32_max(float v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 32));
  return v;
}

template <int DT>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const PackArgs a) {
  __shared__ int32_t row_s[KVQ_GROUP];
  __shared__ uint8_t kcodes_s[KVQ_GROUP * KVQ_MAX_HEAD_DIM];
  __shared__ uint8_t vcodes_s[KVQ_GROUP * KVQ_MAX_HEAD_DIM];

  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int Dk = a.L.Dk, Dv = a.L.Dv;
  const int64_t slab = int64_t(b) * a.L.Hkv + h;
  const RetentionRule rr{a.L.T, a.L.n_recent, a.L.log_window};

  if (int64_t(blockIdx.x) < a.n_groups_chunk) {
    // ------------------------------------------------ one key group of 32 tokens
    const int64_t g = a.g_begin + blockIdx.x;
    if (tid < KVQ_GROUP) row_s[tid] = int32_t(quantized_position(rr, g * KVQ_GROUP + tid) - a.t_begin);
    __syncthreads();

    // keys: thread c owns channel c of all 32 rows
    const float k_levels = float((1 << a.L.k_bits) - 1);
    for (int c = tid; c < Dk; c += kPackThreads) {
      float x[KVQ_GROUP];
      float mn = 0.0f, mx = 0.0f;
#pragma unroll
      for (int t = 0; t < KVQ_GROUP; ++t) {
        x[t] = load_elem<DT>(a.K, (slab * a.t_count + row_s[t]) * Dk + c);
        mn = t == 0 ? x[t] : fminf(mn, x[t]);
        mx = t == 0 ? x[t] : fmaxf(mx, x[t]);
      }
      const QParams q = make_qparams(mn, mx, k_levels);
      const int64_t so = (slab * a.L.n_groups + g) * Dk + c;
      static_cast<uint16_t*>(a.cache.k_scale)[so] = q.s_bits;
      static_cast<uint16_t*>(a.cache.k_zero)[so] = q.z_bits;
#pragma unroll
      for (int t = 0; t < KVQ_GROUP; ++t) kcodes_s[t * Dk + c] = uint8_t(quant_code(x[t], q, k_levels));
    }

    // values: thread c owns channel c; a 32-lane group owns one channel group
    const float v_levels = float((1 << a.L.v_bits) - 1);
    const int ngv = Dv / KVQ_GROUP;
    for (int c = tid; c < Dv; c += kPackThreads) {
      for (int t = 0; t < KVQ_GROUP; ++t) {
        const float x = load_elem<DT>(a.V, (slab * a.t_count + row_s[t]) * Dv + c);
        const float mn = group32_min(x);
        const float mx = group32_max(x);
        const QParams q = make_qparams(mn, mx, v_levels);
        if ((c & (KVQ_GROUP - 1)) == 0) {
          const int64_t so = ((slab * a.L.n_groups + g) * ngv + c / KVQ_GROUP) * KVQ_GROUP + t;
          static_cast<uint16_t*>(a.cache.v_scale)[so] = q.s_bits;
          static_cast<uint16_t*>(a.cache.v_zero)[so] = q.z_bits;
        }
        vcodes_s[t * Dv + c] = uint8_t(quant_code(x, q, v_levels));
      }
    }
    __syncthreads();

    // pack: word w of a row holds channels w*per .. w*per+per-1, code k at bits k*bits
    {
      const int kb = a.L.k_bits, per = 32 / kb, kw = Dk * kb / 32;
      uint32_t* dst = static_cast<uint32_t*>(a.cache.k_codes) + (slab * a.L.Tq + g * KVQ_GROUP) * kw;
      for (int i = tid; i < KVQ_GROUP * kw; i += kPackThreads) {
        const int t = i / kw, w = i - t * kw;
        const uint8_t* src = &kcodes_s[t * Dk + w * per];
        uint32_t word = 0;
        for (int k = 0; k < per; ++k) word |= uint32_t(src[k]) << (k * kb);
        dst[i] = word;
      }
    }
    {
      // values: the group's bit stream of Dv*vb words (layout in kvq_vlayout.hpp);
      // thread i assembles word i from the 32/vb codes it holds
      const int vb = a.L.v_bits, per = 32 / vb, nw = Dv * vb;
      uint32_t* dst = static_cast<uint32_t*>(a.cache.v_codes) + (slab * a.L.n_groups + g) * nw;
      for (int i = tid; i < nw; i += kPackThreads) {
        uint32_t word = 0;
        for (int k = 0; k < per; ++k) {
          const ValueCodeSpot sp = value_code_at(32 * i + k * vb, Dv, vb);
          word |= uint32_t(vcodes_s[sp.tau * Dv + sp.c]) << (k * vb);
        }
        dst[i] = word;
      }
    }
  } else {
    // ------------------------------------------------ retained rows -> fp16
    const int sub = tid / (kPackThreads / kRetRowsPerBlock);
    const int lt = tid % (kPackThreads / kRetRowsPerBlock);
    const int64_t j = (int64_t(blockIdx.x) - a.n_groups_chunk) * kRetRowsPerBlock + sub;
    if (j >= a.n_ret_chunk) return;
    const int64_t r = a.r_begin + j;                       // rank among all retained rows
    const int64_t row = retained_position(rr, r) - a.t_begin;  // row in the chunk
    uint16_t* kd = static_cast<uint16_t*>(a.cache.k_fp16) + (slab * a.L.R + r) * Dk;
    uint16_t* vd = static_cast<uint16_t*>(a.cache.v_fp16) + (slab * a.L.R + r) * Dv;
    for (int c = lt; c < Dk; c += kPackThreads / kRetRowsPerBlock)
      kd[c] = f16_bits_rne(load_elem<DT>(a.K, (slab * a.t_count + row) * Dk + c));
    for (int c = lt; c < Dv; c += kPackThreads / kRetRowsPerBlock)
      vd[c] = f16_bits_rne(load_elem<DT>(a.V, (slab * a.t_count + row) * Dv + c));
  }
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
  const int64_t nblk = a.n_groups_chunk + (a.n_ret_chunk + kRetRowsPerBlock - 1) / kRetRowsPerBlock;
  if (nblk == 0) return hipSuccess;
  const dim3 grid(unsigned(nblk), unsigned(a.L.Hkv), unsigned(a.L.B));
  switch (a.dtype) {
    case KVQ_F32: hipLaunchKernelGGL(pack_kernel<KVQ_F32>, grid, dim3(kPackThreads), 0, stream, a); break;
    case KVQ_F16: hipLaunchKernelGGL(pack_kernel<KVQ_F16>, grid, dim3(kPackThreads), 0, stream, a); break;
    case KVQ_BF16: hipLaunchKernelGGL(pack_kernel<KVQ_BF16>, grid, dim3(kPackThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
