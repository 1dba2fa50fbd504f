// Partition merge of kv_decode_attn: combines the partial results (m, l, o) of
// every query head by log-sum-exp (see kvq_decode_common.hpp) into
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
//
// One workgroup per query head.  Launched on the decode kernel's stream right
// after it, so the partials it reads are complete and visible.  Threads take
// (4-channel quad, partition subset) pairs so every load of the sum is
// independent of the others; the subsets meet in LDS at the end.
#include <hip/hip_runtime.h>

#include "kvq_decode_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int kMergeThreads = 256;

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int tid = threadIdx.x;
  __syncthreads();  // red may still be read by a previous reduction
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__global__ __launch_bounds__(kMergeThreads) void merge_partitions_kernel(const float* partials, int P, int Dv,
                                                                          float* out) {
  __shared__ float red[kMergeThreads / 64];
  __shared__ float4 part_sums[kMergeThreads];
  const int tid = threadIdx.x;
  const int PS = Dv + 4;  // m, l, two unused floats, o[Dv]
  const float* base = partials + int64_t(blockIdx.x) * P * PS;

  float M = -INFINITY;
  for (int p = tid; p < P; p += kMergeThreads) M = fmaxf(M, base[int64_t(p) * PS]);
  M = block_reduce(M, red, true);
  float L = 0.0f;
  for (int p = tid; p < P; p += kMergeThreads) L += lse_weight(base[int64_t(p) * PS], M) * base[int64_t(p) * PS + 1];
  L = block_reduce(L, red, false);

  const int nq = Dv / 4, ns = kMergeThreads / nq;
  const int oq = tid % nq, s = tid / nq;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (s < ns) {
    const float* src = base + 4 + 4 * oq;
    int p = s;
    for (; p + 3 * ns < P; p += 4 * ns) {
      float wt[4];
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = int64_t(p + u * ns) * PS;
        wt[u] = base[row];
        v[u] = *reinterpret_cast<const float4*>(src + row);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = lse_weight(wt[u], M);
        acc.x = fmaf(w, v[u].x, acc.x);
        acc.y = fmaf(w, v[u].y, acc.y);
        acc.z = fmaf(w, v[u].z, acc.z);
        acc.w = fmaf(w, v[u].w, acc.w);
      }
    }
    for (; p < P; p += ns) {
      const int64_t row = int64_t(p) * PS;
      const float w = lse_weight(base[row], M);
      const float4 v = *reinterpret_cast<const float4*>(src + row);
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
  }
  part_sums[tid] = acc;
  __syncthreads();
  if (tid < nq) {
    float4 o = part_sums[tid];
    for (int t = 1; t < ns; ++t) {
      const float4 v = part_sums[t * nq + tid];
      o.x += v.x;
      o.y += v.y;
      o.z += v.z;
      o.w += v.w;
    }
    const float inv = 1.0f / L;
    float4 r;
    r.x = o.x * inv;
    r.y = o.y * inv;
    r.z = o.z * inv;
    r.w = o.w * inv;
    *reinterpret_cast<float4*>(out + int64_t(blockIdx.x) * Dv + 4 * tid) = r;
  }
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int parts, hipStream_t stream) {
  const unsigned rows = unsigned(int64_t(a.L.B) * a.L.Hq);
  hipLaunchKernelGGL(merge_partitions_kernel, dim3(rows), dim3(kMergeThreads), 0, stream, a.partials, parts, a.L.Dv,
                     a.out);
  return hipGetLastError();
}

}  // namespace kvq
