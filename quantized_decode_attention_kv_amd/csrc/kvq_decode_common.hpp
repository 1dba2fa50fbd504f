// Pieces shared by the decode kernels: query loads, the log-sum-exp combination of
// partial softmax states and the cross-partition merge epilogue.
//
// Scores are kept in the log2 domain (s * log2 e) so every exponential is a single
// exp2.  A partial result is (m, l, o): running max m, sum l of 2^(s - m) and the
// unnormalised output o = sum 2^(s - m) v.  Two partials combine as
//   M = max(m1, m2),  l = 2^(m1-M) l1 + 2^(m2-M) l2,  o = 2^(m1-M) o1 + 2^(m2-M) o2,
// which is exact in real arithmetic for any split of the tokens (attention does not
// depend on token order: "LogQuant: Log-Distributed 2-Bit Quantization of KV
// Cache", section 4).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.hpp"

namespace kvq {

// Launch of a decode kernel whose one argument is `a` through hipExtLaunchKernel,
// with a.kernel_start / a.kernel_stop as the start and stop events of that one
// kernel command (the runtime's timing of it).  The callers take this path only
// when one of the two events is set.
inline hipError_t launch_decode_timed(const void* kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                      DecodeArgs a) {
  void* args[] = {&a};
  return hipExtLaunchKernel(kernel, grid, block, args, lds, stream, a.kernel_start, a.kernel_stop, 0);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / 64;

__device__ __forceinline__ float h2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

template <int DT>
__device__ __forceinline__ float load_q(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load_q<KVQ_F32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_q<KVQ_F16>(const void* p, int64_t i) {
  return __half2float(static_cast<const __half*>(p)[i]);
}
template <>
__device__ __forceinline__ float load_q<KVQ_BF16>(const void* p, int64_t i) {
  return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
}

// query element i of a q array of dtype qdt (wave-uniform branch)
__device__ __forceinline__ float load_q_any(const void* p, int qdt, int64_t i) {
  if (qdt == KVQ_BF16) return load_q<KVQ_BF16>(p, i);
  if (qdt == KVQ_F16) return load_q<KVQ_F16>(p, i);
  return load_q<KVQ_F32>(p, i);
}

__device__ __forceinline__ float lse_weight(float m, float M) { return m == -INFINITY ? 0.0f : exp2f(m - M); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Finish one workgroup's (batch b, kv head h, partition p) result for its G query
// heads.  res: LDS [G][Dv + 2] = (m, l, o[Dv]).  P == 1: write out = o / l.
// P > 1: write the partial row (m, l, two unused floats, o[Dv]; o 16-byte
// aligned) for merge_partitions_kernel, launched after this kernel on the same
// stream, to combine.  Plain stores: the kernel boundary makes them visible, so no
// workgroup needs a device-wide fence (each one would write back and invalidate
// the L2 of its XCD).
__device__ inline void finish_partition(const DecodeArgs& a, int G, int b, int h, int p, const float* res) {
  const int tid = threadIdx.x, Dv = a.L.Dv, P = a.P;
  const int64_t qh0 = int64_t(b) * a.L.Hq + int64_t(h) * G;
  if (P == 1) {
    for (int idx = tid; idx < G * Dv; idx += kDecodeThreads) {
      const int i = idx / Dv, c = idx - i * Dv;
      a.out[(qh0 + i) * Dv + c] = res[i * (Dv + 2) + 2 + c] / res[i * (Dv + 2) + 1];
    }
    return;
  }
  const int PS = Dv + 4;
  for (int idx = tid; idx < G * PS; idx += kDecodeThreads) {
    const int i = idx / PS, e = idx - i * PS;
    const float v = e < 2 ? res[i * (Dv + 2) + e] : (e < 4 ? 0.0f : res[i * (Dv + 2) + e - 2]);
    a.partials[((qh0 + i) * P + p) * PS + e] = v;
  }
}

}  // namespace kvq
