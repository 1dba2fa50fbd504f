// Streaming cache: host bookkeeping and the C entry points kvq_stream_* /
// kv_stream_* of include/kvq.h.
//
// One decode-time token per append (LogQuant: Log-Distributed 2-Bit Quantization
// of KV Cache, technical summary, section 2, dynamic adjustment; section 4,
// order-free attention).  Retention depends on positions only, so the state is
// the same for every (batch row, kv head) slab and lives on the host: which fp16
// row holds which position, which rows are pending, how many groups are packed.
// Each append advances it and launches one kernel that applies the step to all
// slabs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "../../include/kvq.h"
#include "kvq_internal.hpp"
#include "kvq_retention.hpp"

namespace {

using kvq::fail;
using kvq::ok;

// Upper bound of the fp16 rows in use at any point of a stream of `capacity`
// tokens: n_recent, plus for every span j that can exist at most W/2 + 1 multiples
// of 2^j in its W 2^(j-1) positions, plus up to 31 pending tokens and the token
// being appended; never more than the capacity.
int64_t row_bound(int64_t n_recent, int64_t W, int64_t capacity) {
  int64_t b = n_recent;
  if (W > 0) {
    for (int j = 1; j < 62 && (W << (j - 1)) < capacity; ++j) b += W / 2 + 1;
  }
  b += KVQ_GROUP;
  return b < capacity ? b : capacity;
}

int check_stream(const kvq_stream* S) {
  if (!S) return fail(KVQ_ERR_INVALID, "stream is NULL");
  const kvq_layout& L = S->L;
  const int st = kvq::check_format(L);
  if (st != KVQ_OK) return st;
  if (L.k_group != KVQ_GROUP) return fail(KVQ_ERR_UNSUPPORTED, "stream key groups are %d tokens", KVQ_GROUP);
  if (L.log_window > 0 && L.n_recent < L.log_window)
    return fail(KVQ_ERR_UNSUPPORTED, "a stream needs log_window == 0 or n_recent (%d) >= log_window (%d)",
                L.n_recent, L.log_window);
  if (S->g_cap != L.T / KVQ_GROUP || S->r_cap != row_bound(L.n_recent, L.log_window, L.T) ||
      S->r_cap > KVQ_STREAM_MAX_ROWS)
    return fail(KVQ_ERR_INVALID, "stream capacities are stale; call kvq_stream_init");
  if (S->t < 0 || S->t > L.T || S->n_groups < 0 || S->n_groups > S->g_cap || S->n_rows < 0 ||
      S->n_rows > S->r_cap || S->n_pending < 0 || S->n_pending >= KVQ_GROUP || S->n_pending > S->n_rows ||
      int64_t(S->n_groups) * KVQ_GROUP + S->n_rows != S->t)
    return fail(KVQ_ERR_INVALID, "stream state is inconsistent (t %d, groups %d, rows %d, pending %d)", S->t,
                S->n_groups, S->n_rows, S->n_pending);
  return KVQ_OK;
}

// One append on the host state: the token's row, the rows that leave the fp16
// set, and the group (with its row moves) once 32 are pending.
int plan_step(kvq_stream& S, kvq_stream_step& step) {
  const kvq_layout& L = S.L;
  if (S.t >= L.T) return fail(KVQ_ERR_INVALID, "stream is full (capacity %d tokens)", L.T);
  if (S.n_rows >= S.r_cap) return fail(KVQ_ERR_INVALID, "fp16 rows exhausted (internal bound %d)", S.r_cap);
  std::memset(&step, 0, sizeof(step));
  step.new_row = S.n_rows;
  step.group = -1;
  S.row_pos[S.n_rows] = S.t;
  S.row_pending[S.n_rows] = 0;
  ++S.n_rows;
  ++S.t;
  for (int i = 0; i < S.n_rows; ++i) {
    if (!S.row_pending[i] && !kvq::retained_at(S.row_pos[i], S.t, L.n_recent, L.log_window)) {
      S.row_pending[i] = 1;
      ++S.n_pending;
    }
  }
  if (S.n_pending < KVQ_GROUP) return KVQ_OK;
  if (S.n_groups >= S.g_cap) return fail(KVQ_ERR_INVALID, "group capacity %d exhausted", S.g_cap);
  // the 32 pending rows of lowest position, in ascending position
  int pend[KVQ_STREAM_MAX_ROWS];
  int np = 0;
  for (int i = 0; i < S.n_rows; ++i)
    if (S.row_pending[i]) pend[np++] = i;
  std::partial_sort(pend, pend + KVQ_GROUP, pend + np,
                    [&](int a, int b) { return S.row_pos[a] < S.row_pos[b]; });
  bool member[KVQ_STREAM_MAX_ROWS] = {};
  step.group = S.n_groups;
  for (int k = 0; k < KVQ_GROUP; ++k) {
    step.member_rows[k] = pend[k];
    step.member_pos[k] = S.row_pos[pend[k]];
    member[pend[k]] = true;
  }
  // keep the rows in use contiguous: rows past the new end move into freed rows
  const int end = S.n_rows - KVQ_GROUP;
  int hole = 0, src = end;
  for (;;) {
    while (hole < end && !member[hole]) ++hole;
    while (src < S.n_rows && member[src]) ++src;
    if (hole >= end || src >= S.n_rows) break;
    step.move_src[step.n_moves] = src;
    step.move_dst[step.n_moves] = hole;
    ++step.n_moves;
    S.row_pos[hole] = S.row_pos[src];
    S.row_pending[hole] = S.row_pending[src];
    ++hole;
    ++src;
  }
  S.n_rows = end;
  S.n_pending -= KVQ_GROUP;
  ++S.n_groups;
  // at most 32 positions leave the set per step, so one group per step suffices
  if (S.n_pending >= KVQ_GROUP) return fail(KVQ_ERR_INVALID, "internal: %d tokens still pending", S.n_pending);
  return KVQ_OK;
}

// Copy of a stream's state limited to the rows in use plus the one an append adds
// (a step only touches rows below n_rows + 1): the row arrays are 20 KB, of which
// a stream uses a few hundred entries.
void copy_state(kvq_stream& dst, const kvq_stream& src) {
  const int rows = std::min<int>(KVQ_STREAM_MAX_ROWS, src.n_rows + 1);
  dst.L = src.L;
  dst.t = src.t;
  dst.n_groups = src.n_groups;
  dst.n_rows = src.n_rows;
  dst.n_pending = src.n_pending;
  dst.g_cap = src.g_cap;
  dst.r_cap = src.r_cap;
  std::memcpy(dst.row_pos, src.row_pos, sizeof(int32_t) * size_t(rows));
  std::memcpy(dst.row_pending, src.row_pending, size_t(rows));
}

int check_stream_cache(const kvq_cache* cache, bool groups) {
  int st;
  if (!cache) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if ((st = kvq::check_cache_ptr(cache->k_fp16, "k_fp16")) || (st = kvq::check_cache_ptr(cache->v_fp16, "v_fp16")))
    return st;
  if (groups) {
    if ((st = kvq::check_cache_ptr(cache->k_codes, "k_codes")) ||
        (st = kvq::check_cache_ptr(cache->k_scale, "k_scale")) ||
        (st = kvq::check_cache_ptr(cache->k_zero, "k_zero")) ||
        (st = kvq::check_cache_ptr(cache->v_codes, "v_codes")) ||
        (st = kvq::check_cache_ptr(cache->v_scale, "v_scale")) || (st = kvq::check_cache_ptr(cache->v_zero, "v_zero")))
      return st;
  }
  return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_stream_init(kvq_stream* S, int B, int Hq, int Hkv, int Dk, int Dv, int capacity, int k_bits, int v_bits,
                    int n_recent, int log_window) {
  return kvq_stream_init_ex(S, B, Hq, Hkv, Dk, Dv, capacity, k_bits, v_bits, n_recent, log_window, KVQ_GROUP);
}

int kvq_stream_init_ex(kvq_stream* S, int B, int Hq, int Hkv, int Dk, int Dv, int capacity, int k_bits, int v_bits,
                       int n_recent, int log_window, int v_group) {
  if (!S) return fail(KVQ_ERR_INVALID, "stream is NULL");
  kvq_layout l{};
  l.B = B;
  l.Hq = Hq;
  l.Hkv = Hkv;
  l.Dk = Dk;
  l.Dv = Dv;
  l.T = capacity;
  l.k_bits = k_bits;
  l.v_bits = v_bits;
  l.n_recent = n_recent;
  l.log_window = log_window;
  l.k_group = KVQ_GROUP;
  l.v_group = v_group;
  int st = kvq::check_format(l);
  if (st != KVQ_OK) return st;
  if (log_window > 0 && n_recent < log_window)
    return fail(KVQ_ERR_UNSUPPORTED, "a stream needs log_window == 0 or n_recent (%d) >= log_window (%d)",
                n_recent, log_window);
  const int64_t rb = row_bound(n_recent, log_window, capacity);
  if (rb > KVQ_STREAM_MAX_ROWS)
    return fail(KVQ_ERR_UNSUPPORTED, "the stream may need %lld fp16 rows, more than %d", (long long)rb,
                KVQ_STREAM_MAX_ROWS);
  std::memset(S, 0, sizeof(*S));
  S->L = l;
  S->g_cap = capacity / KVQ_GROUP;
  S->r_cap = int32_t(rb);
  return ok();
}

int kvq_stream_set_flags(kvq_stream* S, int flags) {
  const int st = check_stream(S);
  if (st != KVQ_OK) return st;
  if (S->t != 0) return fail(KVQ_ERR_INVALID, "flags are set on an empty stream (t is %d)", S->t);
  kvq_layout l = S->L;
  l.flags = flags;
  const int fs = kvq::check_format(l);
  if (fs != KVQ_OK) return fs;
  S->L = l;
  return ok();
}

int kvq_stream_cache_sizes(const kvq_stream* S, size_t bytes_out[KVQ_NUM_CACHE_BUFFERS]) {
  const int st = check_stream(S);
  if (st != KVQ_OK) return st;
  if (!bytes_out) return fail(KVQ_ERR_INVALID, "bytes_out is NULL");
  const kvq_layout& L = S->L;
  const size_t slabs = size_t(L.B) * size_t(L.Hkv), G = size_t(S->g_cap), R = size_t(S->r_cap);
  bytes_out[0] = slabs * G * KVQ_GROUP * size_t(L.Dk * L.k_bits / 32) * 4;  // k_codes
  bytes_out[1] = slabs * G * size_t(L.Dk) * 2;                             // k_scale
  bytes_out[2] = bytes_out[1];                                             // k_zero
  bytes_out[3] = slabs * G * size_t(L.Dv * L.v_bits) * 4;                  // v_codes
  bytes_out[4] = slabs * G * size_t(L.Dv / L.v_group) * KVQ_GROUP * 2;    // v_scale ([Dv/v_group, 32] per group)
  bytes_out[5] = bytes_out[4];                                             // v_zero
  bytes_out[6] = slabs * R * size_t(L.Dk) * 2;                             // k_fp16
  bytes_out[7] = slabs * R * size_t(L.Dv) * 2;                             // v_fp16
  return ok();
}

size_t kvq_stream_workspace_bytes(const kvq_stream* S, int num_partitions) {
  if (check_stream(S) != KVQ_OK || num_partitions < 1 || num_partitions == 1) return 0;
  return kvq::ws_partial_bytes(S->L, num_partitions);
}

int kvq_stream_plan(kvq_stream* S, kvq_stream_step* step) {
  int st = check_stream(S);
  if (st != KVQ_OK) return st;
  if (!step) return fail(KVQ_ERR_INVALID, "step is NULL");
  kvq_stream next;
  copy_state(next, *S);
  st = plan_step(next, *step);
  if (st != KVQ_OK) return st;
  copy_state(*S, next);
  return ok();
}

int kv_stream_prefill(kvq_stream* S, int T0, const void* K, const void* V, int kv_dtype, const kvq_cache* cache,
                      void* stream) {
  int st = check_stream(S);
  if (st != KVQ_OK) return st;
  if (S->t != 0) return fail(KVQ_ERR_INVALID, "prefill needs an empty stream (t = %d)", S->t);
  if (T0 < 1 || T0 > S->L.T) return fail(KVQ_ERR_INVALID, "T0 %d must be in [1, capacity %d]", T0, S->L.T);
  kvq_layout L0 = S->L;
  L0.T = T0;
  const kvq::RetentionRule rule{T0, S->L.n_recent, S->L.log_window};
  const int64_t R = kvq::retained_before(rule, T0), Tq = T0 - R;
  if (Tq % KVQ_GROUP)
    return fail(KVQ_ERR_UNSUPPORTED, "%lld quantized tokens at T0 = %d is not a multiple of 32", (long long)Tq, T0);
  if (R > S->r_cap) return fail(KVQ_ERR_INVALID, "internal: %lld retained rows exceed the bound %d", (long long)R, S->r_cap);
  L0.R = int32_t(R);
  L0.Tq = int32_t(Tq);
  L0.n_groups = int32_t(Tq / KVQ_GROUP);
  if (L0.n_recent > T0) L0.n_recent = T0;  // the rule keeps at most all T0 tokens either way
  st = kvq::pack_view(L0, S->g_cap, S->r_cap, 0, T0, K, V, kv_dtype, cache, stream);
  if (st != KVQ_OK) return st;
  S->t = T0;
  S->n_groups = L0.n_groups;
  S->n_rows = 0;
  S->n_pending = 0;
  for (int64_t p = 0; p < T0; ++p) {
    if (kvq::retained_at(p, T0, S->L.n_recent, S->L.log_window)) {
      S->row_pos[S->n_rows] = int32_t(p);
      S->row_pending[S->n_rows] = 0;
      ++S->n_rows;
    }
  }
  return ok();
}

int kv_stream_append(kvq_stream* S, const void* k_new, const void* v_new, int kv_dtype, const kvq_cache* cache,
                     void* stream) {
  int st = check_stream(S);
  if (st != KVQ_OK) return st;
  if (!kvq::valid_dtype(kv_dtype)) return fail(KVQ_ERR_INVALID, "kv_dtype %d is not KVQ_F32/F16/BF16", kv_dtype);
  if (!k_new || !v_new) return fail(KVQ_ERR_INVALID, "k_new or v_new is NULL");
  if (!kvq::aligned16(k_new) || !kvq::aligned16(v_new))
    return fail(KVQ_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  kvq_stream next;
  copy_state(next, *S);
  kvq_stream_step step;
  st = plan_step(next, step);
  if (st != KVQ_OK) return st;
  if ((st = check_stream_cache(cache, step.group >= 0)) != KVQ_OK) return st;
  kvq::AppendArgs a{};
  a.L = S->L;
  a.g_stride = S->g_cap;
  a.r_stride = S->r_cap;
  a.k_new = k_new;
  a.v_new = v_new;
  a.dtype = kv_dtype;
  a.new_row = step.new_row;
  a.group = step.group;
  for (int k = 0; k < KVQ_GROUP; ++k) {
    a.member_rows[k] = step.member_rows[k];
    a.move_src[k] = step.move_src[k];
    a.move_dst[k] = step.move_dst[k];
  }
  a.n_moves = step.n_moves;
  a.cache = *cache;
  const hipError_t e = kvq::launch_append(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  copy_state(*S, next);
  return ok();
}

int kv_stream_decode(const kvq_stream* S, const void* q, int q_dtype, const kvq_cache* cache, float softmax_scale,
                     int num_partitions, void* workspace, size_t workspace_bytes, float* out, void* stream) {
  const int st = check_stream(S);
  if (st != KVQ_OK) return st;
  if (S->t < 1) return fail(KVQ_ERR_INVALID, "stream is empty");
  kvq_layout Lv = S->L;
  Lv.T = S->t;
  Lv.R = S->n_rows;
  Lv.n_groups = S->n_groups;
  Lv.Tq = S->n_groups * KVQ_GROUP;
  return kvq::decode_view(Lv, S->g_cap, S->r_cap, q, q_dtype, cache, softmax_scale, num_partitions, workspace,
                          workspace_bytes, out, stream, nullptr);
}

}  // extern "C"
