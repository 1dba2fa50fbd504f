// Retention rule shared by host validation and device kernels of the library.
//
// Which cached positions stay in fp16 (LogQuant: Log-Distributed 2-Bit Quantization
// of KV Cache, technical summary section 2, log-based filtering): the newest
// n_recent positions, and for W = log_window > 0 and j = 1, 2, ... the multiples of
// 2^j inside [T - W*2^j, T - W*2^(j-1)) clipped at 0.  Everything here is closed
// form in the position, so a kernel can find the positions of any key group or
// retained row without a lookup table.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct RetentionRule {
  int64_t T, n_recent, W;
};

__host__ __device__ inline int64_t ceil_div_nonneg(int64_t a, int64_t m) { return (a + m - 1) / m; }

// Number of retained positions in [0, p), 0 <= p <= T.
__host__ __device__ inline int64_t retained_before(const RetentionRule& r, int64_t p) {
  int64_t win0 = r.T - r.n_recent;
  if (win0 < 0) win0 = 0;
  int64_t cnt = p > win0 ? p - win0 : 0;
  if (r.W > 0) {
    for (int j = 1; j < 62; ++j) {
      const int64_t hi = r.T - (r.W << (j - 1));
      if (hi <= 0) break;
      int64_t lo = r.T - (r.W << j);
      if (lo < 0) lo = 0;
      int64_t e = hi < win0 ? hi : win0;  // positions at or after win0 are already counted
      if (e > p) e = p;
      if (e > lo) {
        const int64_t m = int64_t(1) << j;
        cnt += ceil_div_nonneg(e, m) - ceil_div_nonneg(lo, m);
      }
    }
  }
  return cnt;
}

__host__ __device__ inline int64_t quantized_before(const RetentionRule& r, int64_t p) {
  return p - retained_before(r, p);
}

// Position of the k-th quantized position (0 <= k < Tq): the smallest p with
// quantized_before(p + 1) > k.
__host__ __device__ inline int64_t quantized_position(const RetentionRule& r, int64_t k) {
  int64_t lo = k, hi = r.T - 1;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (quantized_before(r, mid + 1) > k) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Position of the k-th retained position (0 <= k < R).
__host__ __device__ inline int64_t retained_position(const RetentionRule& r, int64_t k) {
  int64_t lo = k, hi = r.T - 1;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (retained_before(r, mid + 1) > k) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Whether position p (0 <= p < t) is retained when the cache holds t tokens (the
// rule above with T = t, per position): the newest n_recent, else with W > 0 the
// span j >= 1 holding the distance d = t - p (W 2^(j-1) < d <= W 2^j) keeps the
// multiples of 2^j.
__host__ __device__ inline bool retained_at(int64_t p, int64_t t, int64_t n_recent, int64_t W) {
  const int64_t d = t - p;
  if (d <= n_recent) return true;
  if (W <= 0 || d <= W) return false;
  int j = 1;
  while ((W << j) < d) ++j;
  return (p & ((int64_t(1) << j) - 1)) == 0;
}

}  // namespace kvq
