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
  int64_t g_stride, r_stride;        // key groups / fp16 rows per slab in the cache arrays
  const void* K;
  const void* V;
  int dtype;
  kvq_cache cache;
};

constexpr int kMaxTeamTable = 128;  // teams per slab whose run starts travel with the launch

struct DecodeArgs {
  kvq_layout L;
  const void* q;
  int q_dtype;
  kvq_cache cache;
  float scale;
  int P;
  int64_t g_stride, r_stride;  // key groups / fp16 rows per slab in the cache arrays (>= n_groups, R)
  int units;           // work units per slab of the matrix-core kernel (set by its launcher)
  int ranks;           // waves per SIMD the matrix-core grid puts on the device at once (1..4)
  // first key group of each team's run, teams 0 .. T (set by the matrix-core
  // launcher on the host when T <= kMaxTeamTable; n_team_first = 0: the kernel
  // computes them itself)
  int n_team_first;
  int team_first[kMaxTeamTable + 1];
  float* partials;     // [B * Hq, units, Dv + 4]: m (log2 domain), l, 2 unused, unnormalised o (P > 1)
  float* out;          // [B, Hq, Dv]
  // HeadQ side code (side_rank == 0: none; the vector-ALU kernel then adds the
  // logit correction (U^T q) . z_hat per quantized token)
  const float* side_u;        // [Hkv, Dk, side_rank]
  const uint8_t* side_codes;  // [B, Hkv, g_stride * 32, side_rank]
  const uint16_t* side_scale; // [B, Hkv, g_stride * 32] fp16
  const uint16_t* side_zero;
  int side_rank;
  // host side only: timing events of the decode kernel's own dispatch (null: none)
  hipEvent_t kernel_start, kernel_stop;
};

// Side-code write of the HeadQ mechanics: one workgroup per (code group, kv head, batch)
struct SideArgs {
  kvq_layout L;
  const void* K;  // [B, Hkv, T, Dk] in dtype
  int dtype;
  kvq_cache cache;
  const float* U;  // [Hkv, Dk, rank]
  int rank, bits;
  uint8_t* codes;
  uint16_t* scale;
  uint16_t* zero;
};
hipError_t launch_side_pack(const SideArgs& a, hipStream_t stream);
constexpr int kMaxSideRank = 16;

// Work units of the matrix-core decode kernel: each of the P split-K partitions
// is cut into c = 1, 2, 4 or 8 units, one wave each (four independent waves share
// a workgroup, one per SIMD of a compute unit).  c
// is the largest that keeps the grid within `resident` waves (what the device
// holds at once for the kernel's occupancy), so short caches still fill the chip
// while long ones keep each wave on a long run of key groups.  P == 1 is one
// unit, which writes the output directly.
constexpr int kMaxUnitsPerPartition = 8;
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

// One streaming append on the device (kv_stream_append): one workgroup per slab
// writes the token's fp16 row, packs the group the step forms (if any) from its
// fp16 rows and moves rows into the freed ones, in that order.
struct AppendArgs {
  kvq_layout L;                 // format (B, Hkv, Dk, Dv, bits)
  int64_t g_stride, r_stride;   // group / fp16-row capacity per slab
  const void* k_new;            // [B, Hkv, Dk] of dtype
  const void* v_new;            // [B, Hkv, Dv] of dtype
  int dtype;
  int new_row;                  // row of the appended token
  int group;                    // group formed, -1 for none
  int member_rows[KVQ_GROUP];   // its tokens' rows, ascending position
  int n_moves;
  int move_src[KVQ_GROUP], move_dst[KVQ_GROUP];
  kvq_cache cache;
};

hipError_t launch_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// Device address of the static scratch array on the current device (looked up
// once per device; kv_decode_attn_noalloc).
hipError_t static_scratch(void** ptr);

// Current device and its compute-unit count (the attribute is read once per device
// and kept).
hipError_t device_cus(int* dev, int* cus);

// How a decode request is carried out: which kernel, how many partial rows each
// query head gets (the merge folds them; 1 = the decode kernel writes the output),
// the matrix-core kernel's LDS ring depth and its grid.
struct DecodePlan {
  int kernel;       // KVQ_KERNEL_MFMA or KVQ_KERNEL_VALU
  int units;        // work units per (batch, KV head) slab
  int rows;         // partial rows per query head that the merge combines (1: none)
  int depth;        // key groups in a wave's LDS ring (matrix-core kernel), else 0
  int ranks;        // waves per SIMD of the matrix-core grid, else 0
  int64_t waves;    // waves the decode kernel launches
};
// Shapes the matrix-core kernel takes: 4 query heads per KV head, value width 128,
// key width 32, 64 or 128, 2/4/8-bit codes with at least 4 key-code bytes per lane
// and a tile row, per-slab offsets inside 32 bits.  Everything else runs on the
// vector-ALU kernel; a request the matrix-core kernel takes never falls back.
bool mfma_takes(const kvq_layout& L, int P);
// Matrix-core kernel: fill *plan and, when `launch`, enqueue the kernel.
hipError_t mfma_decode(const DecodeArgs& a, hipStream_t stream, DecodePlan* plan, bool launch);
// The plan of a request (a.L, a.P, a.side_rank are read).
hipError_t plan_decode(const DecodeArgs& a, DecodePlan* plan);
// Bytes of partial rows a planned decode writes (0 when units == 1).
// (sized by the unit count, an upper bound of the rows the kernels write)
inline size_t plan_partial_bytes(const kvq_layout& L, const DecodePlan& p) {
  return p.units <= 1 ? 0 : size_t(L.B) * size_t(L.Hq) * size_t(p.units) * size_t(L.Dv + 4) * sizeof(float);
}
// Decode kernel of `plan` followed, when plan.rows > 1, by the partition merge;
// after_decode (if not null) is recorded on the stream between the two.
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream, hipEvent_t after_decode);

// Host helpers of the C ABI layer (kvq_api.cpp), shared with the streaming
// entry points (kvq_stream.cpp).
int fail(int status, const char* fmt, ...);  // sets the thread's last-error text, returns status
int ok();                                     // clears it, returns KVQ_OK
inline bool valid_bits(int b) { return b == 1 || b == 2 || b == 3 || b == 4 || b == 8; }
inline bool valid_gqa(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }
inline bool valid_dtype(int d) { return d == KVQ_F32 || d == KVQ_F16 || d == KVQ_BF16; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int check_cache_ptr(const void* p, const char* name);
int check_format(const kvq_layout& L);
int pack_view(const kvq_layout& L, int64_t g_stride, int64_t r_stride, int64_t t_begin, int64_t t_count,
              const void* K, const void* V, int kv_dtype, const kvq_cache* cache, void* stream);
int decode_view(const kvq_layout& L, int64_t g_stride, int64_t r_stride, const void* q, int q_dtype,
                const kvq_cache* cache, float softmax_scale, int num_partitions, void* workspace,
                size_t workspace_bytes, float* out, void* stream, void* event_after_decode,
                const DecodeArgs* side = nullptr, int workspace_short_status = KVQ_ERR_INVALID,
                void* kernel_start = nullptr, void* kernel_stop = nullptr);

}  // namespace kvq
