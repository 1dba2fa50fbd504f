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
  float* partials;     // [B * Hq, P, Dv + 4]: m (log2 domain), l, 2 unused, unnormalised o (P > 1)
  float* out;          // [B, Hq, Dv]
};

// Workspace of kv_decode_attn: the per-partition partial results.
inline size_t ws_partial_bytes(const kvq_layout& L, int P) {
  return size_t(L.B) * size_t(L.Hq) * size_t(P) * size_t(L.Dv + 4) * sizeof(float);
}

hipError_t launch_pack(const PackArgs& a, hipStream_t stream);
// Decode kernel (matrix-core kernel where it applies, else the generic one)
// followed, when P > 1, by the partition merge.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace kvq
