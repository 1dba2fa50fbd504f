// kv_stream_append kernel for gfx950: one decode-time token into a streaming cache.
//
// LogQuant: Log-Distributed 2-Bit Quantization of KV Cache (technical summary,
// section 2, dynamic adjustment; section 4, order-free attention).  The host
// decides what a step does (the same for every slab); one workgroup per (batch
// row, kv head) slab then
//   1. writes the token's fp16 row (round to nearest even);
//   2. when a group forms, quantizes its 32 fp16 rows with the quantizer contract
//      of kvq.h: keys per channel over the 32 tokens, values per token over each
//      v_group-channel group, codes in the group formats of kvq.h;
//   3. moves fp16 rows past the new end into the rows the group freed.
// With key rotation the token's key row is rotated first (Walsh-Hadamard, the
// butterfly order of kvq.h, through LDS), so its fp16 row and the groups formed
// from such rows hold rotated keys.
// The appended token's values are taken from the input wherever step 2 or 3
// needs them, so no thread reads what another thread of the launch has stored.
// This is a latency-bound launch (a few KB per slab): 1024 threads per slab keep
// the dependent chains short (4 key tokens and 4 value elements per thread).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.hpp"
#include "kvq_rotate.hpp"
#include "kvq_vlayout.hpp"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kAppendThreads = 1024;
constexpr int kSlices = 8;  // key token slices of 4 tokens: (channel, slice) per thread
constexpr int kMaxValuesPerThread = KVQ_GROUP * KVQ_MAX_HEAD_DIM / kAppendThreads;

__device__ inline float load_as_f32(const void* p, int dtype, int64_t i) {
  if (dtype == KVQ_F32) return static_cast<const float*>(p)[i];
  if (dtype == KVQ_F16) return __half2float(static_cast<const __half*>(p)[i]);
  return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);  // bf16
}
__device__ inline uint16_t to_f16_bits(float x) { return __half_as_ushort(__float2half_rn(x)); }
__device__ inline float f16_to_f32(uint16_t b) { return __half2float(__ushort_as_half(b)); }

struct Quant {
  float s, z;
  uint16_t sb, zb;
};

// s = fp16(fp32(mx - mn) / (2^bits - 1)), z = fp16(mn), a zero of either sign
// stored as +0
__device__ inline Quant quant_params(float mn, float mx, float levels) {
  Quant q;
  q.sb = to_f16_bits((mx - mn) / levels);
  q.zb = to_f16_bits(mn);
  if ((q.sb & 0x7fffu) == 0) q.sb = 0;
  if ((q.zb & 0x7fffu) == 0) q.zb = 0;
  q.s = f16_to_f32(q.sb);
  q.z = f16_to_f32(q.zb);
  return q;
}

// code = clamp(rint((x - z) / s), 0, levels) with the correctly rounded division;
// 0 when s == 0
__device__ inline uint32_t quant_code(float x, const Quant& q, float levels) {
  if (q.s == 0.0f) return 0u;
  const float t = __builtin_rintf((x - q.z) / q.s);
  return uint32_t(fminf(fmaxf(t, 0.0f), levels));
}

// OR a 3-bit code into LDS words at stream bit `bit`, into the next word too when
// it straddles
__device__ __forceinline__ void or_code3(uint32_t* w, int bit, uint32_t code) {
  const int sh = bit & 31;
  atomicOr(&w[bit >> 5], code << sh);
  if (sh > 29) atomicOr(&w[(bit >> 5) + 1], code >> (32 - sh));
}

template <int KB, int VB>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  __shared__ uint32_t vw[KVQ_MAX_HEAD_DIM * VB];             // value code words of the group
  // 3-bit key rows are bit streams whose codes may straddle words: built in LDS
  __shared__ uint32_t kw3[KB == 3 ? KVQ_GROUP * KVQ_MAX_HEAD_DIM * 3 / 32 : 1];
  __shared__ float kmn[kSlices][KVQ_MAX_HEAD_DIM], kmx[kSlices][KVQ_MAX_HEAD_DIM];
  __shared__ float vmn[KVQ_GROUP][KVQ_MAX_HEAD_DIM / 32], vmx[KVQ_GROUP][KVQ_MAX_HEAD_DIM / 32];
  const int64_t slab = blockIdx.x;
  const int tid = threadIdx.x;
  const int Dk = a.L.Dk, Dv = a.L.Dv;
  uint16_t* kf = static_cast<uint16_t*>(a.cache.k_fp16) + slab * a.r_stride * Dk;
  uint16_t* vf = static_cast<uint16_t*>(a.cache.v_fp16) + slab * a.r_stride * Dv;
  // rotated keys: the token's rotated key row in fp16, formed by all threads before
  // the first use (one butterfly h per pass, partner channel c ^ h)
  __shared__ float krot[KVQ_MAX_HEAD_DIM];
  __shared__ uint16_t knew16[KVQ_MAX_HEAD_DIM];
  const bool rot = (a.L.flags & KVQ_KEY_ROTATION) != 0;  // the same for every thread
  if (rot) {
    float x = tid < Dk ? load_as_f32(a.k_new, a.dtype, slab * Dk + tid) : 0.0f;
    for (int hh = 1; hh < Dk; hh <<= 1) {
      if (tid < Dk) krot[tid] = x;
      __syncthreads();
      const float partner = tid < Dk ? krot[tid ^ hh] : 0.0f;
      __syncthreads();
      x = butterfly(x, partner, (tid & hh) != 0);
    }
    if (tid < Dk) knew16[tid] = to_f16_bits(rotation_scaled(x, rotation_scale(31 - __builtin_clz(unsigned(Dk)))));
    __syncthreads();
  }
  // the appended token's fp16 value of key / value channel c
  auto k_new16 = [&](int c) {
    return rot ? knew16[c] : to_f16_bits(load_as_f32(a.k_new, a.dtype, slab * Dk + c));
  };
  auto v_new16 = [&](int c) { return to_f16_bits(load_as_f32(a.v_new, a.dtype, slab * Dv + c)); };

  // 1. the token's row
  if (tid < Dk) kf[int64_t(a.new_row) * Dk + tid] = k_new16(tid);
  if (tid < Dv) vf[int64_t(a.new_row) * Dv + tid] = v_new16(tid);
  if (a.group < 0) return;  // the same for every thread: no barrier below is reached

  // 2. the group
  for (int i = tid; i < Dv * VB; i += kAppendThreads) vw[i] = 0u;
  if constexpr (KB == 3) {
    for (int i = tid; i < KVQ_GROUP * Dk * 3 / 32; i += kAppendThreads) kw3[i] = 0u;
  }
  const int64_t gi = slab * a.g_stride + a.group;
  auto k_row = [&](int j, int c) {
    const int row = a.member_rows[j];
    return f16_to_f32(row == a.new_row ? k_new16(c) : kf[int64_t(row) * Dk + c]);
  };
  auto v_row = [&](int j, int c) {
    const int row = a.member_rows[j];
    return f16_to_f32(row == a.new_row ? v_new16(c) : vf[int64_t(row) * Dv + c]);
  };
  constexpr float klev = float((1 << KB) - 1), vlev = float((1 << VB) - 1);
  constexpr int per = 32 / KB;  // key codes per word
  const int kwords = Dk * KB / 32;
  // keys: thread (channel c, slice sl) holds tokens 4 sl .. 4 sl + 3 of channel c;
  // the slices' minima and maxima meet in LDS.  Dk is a multiple of 32, so the
  // `per` channels of a code word are adjacent lanes of one wave.
  constexpr int kMaxKeyPasses = KVQ_MAX_HEAD_DIM * kSlices / kAppendThreads;
  float kx[kMaxKeyPasses][4];
#pragma unroll
  for (int pass = 0; pass < kMaxKeyPasses; ++pass) {
    const int u = tid + pass * kAppendThreads;
    if (u < Dk * kSlices) {
      const int sl = u / Dk, c = u - sl * Dk;
      float mn = INFINITY, mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        kx[pass][k] = k_row(4 * sl + k, c);
        mn = fminf(mn, kx[pass][k]);
        mx = fmaxf(mx, kx[pass][k]);
      }
      kmn[sl][c] = mn;
      kmx[sl][c] = mx;
    }
  }
  __syncthreads();
  uint32_t* kc = static_cast<uint32_t*>(a.cache.k_codes) + gi * KVQ_GROUP * kwords;
#pragma unroll
  for (int pass = 0; pass < kMaxKeyPasses; ++pass) {
    const int u = tid + pass * kAppendThreads;
    if (u < Dk * kSlices) {
      const int sl = u / Dk, c = u - sl * Dk;
      float mn = kmn[0][c], mx = kmx[0][c];
#pragma unroll
      for (int i = 1; i < kSlices; ++i) {
        mn = fminf(mn, kmn[i][c]);
        mx = fmaxf(mx, kmx[i][c]);
      }
      const Quant q = quant_params(mn, mx, klev);
      if (sl == 0) {
        static_cast<uint16_t*>(a.cache.k_scale)[gi * Dk + c] = q.sb;
        static_cast<uint16_t*>(a.cache.k_zero)[gi * Dk + c] = q.zb;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (KB == 3) {
          or_code3(kw3 + (4 * sl + k) * kwords, 3 * c, quant_code(kx[pass][k], q, klev));
        } else {
          uint32_t w = quant_code(kx[pass][k], q, klev) << ((c % per) * KB);
#pragma unroll
          for (int o = 1; o < per; o <<= 1) w |= uint32_t(__shfl_xor(int(w), o));
          if (c % per == 0) kc[(4 * sl + k) * kwords + c / per] = w;
        }
      }
    }
  }
  // values: element e = tid + 1024 i = (token j, channel c), Dv / 32 per thread.
  // Minima and maxima over each 32-channel chunk (32 adjacent lanes) with lane
  // exchanges, then over the v_group / 32 chunks of a group through LDS; codes are
  // OR-ed into the group's bit stream in LDS.
  const int vg = a.L.v_group, nve = KVQ_GROUP * Dv / kAppendThreads;
  float vx[kMaxValuesPerThread];
#pragma unroll
  for (int i = 0; i < kMaxValuesPerThread; ++i) {
    if (i < nve) {  // the same for every thread
      const int e = tid + i * kAppendThreads, j = e / Dv, c = e - j * Dv;
      vx[i] = v_row(j, c);
      float mn = vx[i], mx = vx[i];
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
      }
      if ((c & 31) == 0) {
        vmn[j][c >> 5] = mn;
        vmx[j][c >> 5] = mx;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMaxValuesPerThread; ++i) {
    if (i < nve) {
      const int e = tid + i * kAppendThreads, j = e / Dv, c = e - j * Dv;
      const int g = c / vg, c0 = g * (vg >> 5);
      float mn = vmn[j][c0], mx = vmx[j][c0];
      for (int k = 1; k < (vg >> 5); ++k) {
        mn = fminf(mn, vmn[j][c0 + k]);
        mx = fmaxf(mx, vmx[j][c0 + k]);
      }
      const Quant q = quant_params(mn, mx, vlev);
      if (c == g * vg) {
        const int64_t si = (gi * (Dv / vg) + g) * KVQ_GROUP + j;
        static_cast<uint16_t*>(a.cache.v_scale)[si] = q.sb;
        static_cast<uint16_t*>(a.cache.v_zero)[si] = q.zb;
      }
      const int bit = value_bit_position(j, c, Dv, VB);
      if constexpr (VB == 3)
        or_code3(vw, bit, quant_code(vx[i], q, vlev));
      else
        atomicOr(&vw[bit >> 5], quant_code(vx[i], q, vlev) << (bit & 31));
    }
  }
  __syncthreads();  // the group's rows have been read and its value words are complete
  uint32_t* vc = static_cast<uint32_t*>(a.cache.v_codes) + gi * (Dv * VB);
  for (int i = tid; i < Dv * VB; i += kAppendThreads) vc[i] = vw[i];
  if constexpr (KB == 3) {
    for (int i = tid; i < KVQ_GROUP * kwords; i += kAppendThreads) kc[i] = kw3[i];
  }

  // 3. moves: sources lie past the new end, destinations are freed rows
  for (int e = tid; e < a.n_moves * Dk; e += kAppendThreads) {
    const int m = e / Dk, c = e - m * Dk;
    const int src = a.move_src[m];
    kf[int64_t(a.move_dst[m]) * Dk + c] = src == a.new_row ? k_new16(c) : kf[int64_t(src) * Dk + c];
  }
  for (int e = tid; e < a.n_moves * Dv; e += kAppendThreads) {
    const int m = e / Dv, c = e - m * Dv;
    const int src = a.move_src[m];
    vf[int64_t(a.move_dst[m]) * Dv + c] = src == a.new_row ? v_new16(c) : vf[int64_t(src) * Dv + c];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t slabs = int64_t(a.L.B) * a.L.Hkv;
  if (slabs < 1 || slabs > 0x7fffffff) return hipErrorInvalidValue;
  const int kb = a.L.k_bits, vb = a.L.v_bits;
#define KVQ_APPEND_CASE(K_, V_)                                                                      \
  if (kb == K_ && vb == V_) {                                                                        \
    hipLaunchKernelGGL((append_kernel<K_, V_>), dim3(unsigned(slabs)), dim3(kAppendThreads), 0, stream, a); \
    return hipGetLastError();                                                                        \
  }
  KVQ_APPEND_CASE(1, 1) KVQ_APPEND_CASE(1, 2) KVQ_APPEND_CASE(1, 4) KVQ_APPEND_CASE(1, 8)
  KVQ_APPEND_CASE(2, 1) KVQ_APPEND_CASE(2, 2) KVQ_APPEND_CASE(2, 4) KVQ_APPEND_CASE(2, 8)
  KVQ_APPEND_CASE(4, 1) KVQ_APPEND_CASE(4, 2) KVQ_APPEND_CASE(4, 4) KVQ_APPEND_CASE(4, 8)
  KVQ_APPEND_CASE(8, 1) KVQ_APPEND_CASE(8, 2) KVQ_APPEND_CASE(8, 4) KVQ_APPEND_CASE(8, 8)
  KVQ_APPEND_CASE(3, 1) KVQ_APPEND_CASE(3, 2) KVQ_APPEND_CASE(3, 3) KVQ_APPEND_CASE(3, 4) KVQ_APPEND_CASE(3, 8)
  KVQ_APPEND_CASE(1, 3) KVQ_APPEND_CASE(2, 3) KVQ_APPEND_CASE(4, 3) KVQ_APPEND_CASE(8, 3)
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
