// Partition merge of kv_decode_attn: combines the partial results (m, l, o) of
// every query head by log-sum-exp (see kvq_decode_common.hpp) into
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
//
// One workgroup per query head.  Launched on the decode kernel's stream right
// after it, so the partials it reads are complete and visible.  Threads take
// (4-channel quad, partition subset) pairs and fold their partitions with the
// same rule in a single pass (so the partials are read in one round of loads,
// not one for the maximum, one for the sum and one for the output); the subsets
// meet in LDS at the end.
#include <hip/hip_runtime.h>

#include "kvq_decode_common.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void merge_partitions_kernel(const float* partials, int P, int Dv,
                                                                          float* out) {
  __shared__ float4 part_o[kMergeThreads];
  __shared__ float part_m[kMergeThreads], part_l[kMergeThreads];
  const int tid = threadIdx.x;
  const int PS = Dv + 4;  // m, l, two unused floats, o[Dv]
  const float* base = partials + int64_t(blockIdx.x) * P * PS;

  // thread (quad oq, subset s) folds partitions s, s + ns, ... into its own
  // (max, sum, output) with the log-sum-exp rule: one pass over the partials, all
  // loads of a step independent
  const int nq = Dv / 4, ns = kMergeThreads / nq;
  const int oq = tid % nq, s = tid / nq;
  float mt = -INFINITY, lt = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  auto fold = [&](float mp, float lp, float4 v) {
    if (mp > mt) {  // the running maximum moves: rescale what is held
      const float r = lse_weight(mt, mp);
      acc.x *= r;
      acc.y *= r;
      acc.z *= r;
      acc.w *= r;
      lt *= r;
      mt = mp;
    }
    const float w = lse_weight(mp, mt);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
    lt = fmaf(w, lp, lt);
  };
  if (s < ns) {
    const float* src = base + 4 + 4 * oq;
    int p = s;
    for (; p + 3 * ns < P; p += 4 * ns) {
      float2 ml[4];
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = int64_t(p + u * ns) * PS;
        ml[u] = *reinterpret_cast<const float2*>(base + row);
        v[u] = *reinterpret_cast<const float4*>(src + row);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) fold(ml[u].x, ml[u].y, v[u]);
    }
    for (; p < P; p += ns) {
      const int64_t row = int64_t(p) * PS;
      const float2 ml = *reinterpret_cast<const float2*>(base + row);
      fold(ml.x, ml.y, *reinterpret_cast<const float4*>(src + row));
    }
  }
  part_o[tid] = acc;
  part_m[tid] = mt;
  part_l[tid] = lt;
  __syncthreads();
  if (tid < nq) {
    // the subsets of this quad; every quad of a subset holds the same (max, sum)
    float M = part_m[tid];
    for (int t = 1; t < ns; ++t) M = fmaxf(M, part_m[t * nq + tid]);
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float L = 0.0f;
    for (int t = 0; t < ns; ++t) {
      const int i = t * nq + tid;
      const float w = lse_weight(part_m[i], M);
      const float4 v = part_o[i];
      o.x = fmaf(w, v.x, o.x);
      o.y = fmaf(w, v.y, o.y);
      o.z = fmaf(w, v.z, o.z);
      o.w = fmaf(w, v.w, o.w);
      L = fmaf(w, part_l[i], L);
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
