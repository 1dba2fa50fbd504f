// Internal launch interface between the C ABI layer (kvq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

// Everything a pack launch needs, validated by the caller.
struct PackArgs {
  kvq_layout L;
  int64_t t_begin, t_count;
  int64_t g_begin, n_groups_chunk;   // key groups the chunk owns
  int64_t r_begin, n_ret_chunk;      // retained rows the chunk owns
  const void* K;
  const void* V;
  int dtype;
  kvq_cache cache;
};

struct DecodeArgs {
  kvq_layout L;
  const void* q;
  int q_dtype;
  kvq_cache cache;
  float scale;
  int P;
  int units;           // work units per slab of the matrix-core kernel (set by its launcher)
  int ranks;           // waves per SIMD the matrix-core grid puts on the device at once (1..4)
  float* partials;     // [B * Hq, units, Dv + 4]: m (log2 domain), l, 2 unused, unnormalised o (P > 1)
  float* out;          // [B, Hq, Dv]
};

// Work units of the matrix-core decode kernel: each of the P split-K partitions
// is cut into c = 1, 2 or 4 contiguous runs, one single-wave workgroup each.  c
// is the largest that keeps the grid within `resident` waves (what the device
// holds at once for the kernel's occupancy), so short caches still fill the chip
// while long ones keep each wave on a long run of key groups.  P == 1 is one
// unit, which writes the output directly.
constexpr int kMaxUnitsPerPartition = 4;
inline int decode_mfma_units(const kvq_layout& L, int P, int64_t resident) {
  if (P == 1) return 1;
  const int64_t slabs = int64_t(L.B) * L.Hkv;
  int c = kMaxUnitsPerPartition;
  while (c > 1 && slabs * P * c > resident) c >>= 1;
  return c * P;
}

// Workspace of kv_decode_attn: partial results, one row of Dv + 4 floats per
// (query head, work unit); sized for the largest unit count of the matrix-core
// kernel (the generic kernel writes one row per partition).
inline size_t ws_partial_bytes(const kvq_layout& L, int P) {
  const size_t units = P == 1 ? 0 : size_t(kMaxUnitsPerPartition) * size_t(P);
  return size_t(L.B) * size_t(L.Hq) * units * size_t(L.Dv + 4) * sizeof(float);
}

hipError_t launch_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
// Decode kernel (matrix-core kernel where it applies, else the generic one)
// followed, when P > 1, by the partition merge; after_decode (if not null) is
// recorded on the stream between the two.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t after_decode);

}  // namespace kvq
