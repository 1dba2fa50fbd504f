// C ABI of the library: argument validation, size queries and launches.
// Every check runs on the host before any HIP call, so invalid requests never
// reach the GPU.  See include/kvq.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/kvq.h"
#include "kvq_internal.hpp"
#include "kvq_retention.hpp"

namespace {

thread_local char g_last_error[512] = "";

}  // namespace

int kvq::fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int kvq::ok() {
  g_last_error[0] = '\0';
  return KVQ_OK;
}

namespace {

using kvq::fail;
using kvq::ok;

using kvq::aligned16;
using kvq::valid_bits;
using kvq::valid_gqa;

kvq::RetentionRule rule_of(const kvq_layout& L) { return kvq::RetentionRule{L.T, L.n_recent, L.log_window}; }

// Full validation of a layout (also of one the caller may have edited by hand).
int check_layout(const kvq_layout* L) {
  if (!L) return fail(KVQ_ERR_INVALID, "layout is NULL");
  const int st = kvq::check_format(*L);
  if (st != KVQ_OK) return st;
  const int64_t R = kvq::retained_before(rule_of(*L), L->T);
  const int64_t Tq = L->T - R;
  if (Tq % L->k_group != 0)
    return fail(KVQ_ERR_UNSUPPORTED,
                "%lld quantized tokens is not a multiple of the key group (%d); adjust n_recent so T - R is",
                (long long)Tq, L->k_group);
  if (L->R != R || L->Tq != Tq || L->n_groups != Tq / KVQ_GROUP)
    return fail(KVQ_ERR_INVALID, "layout derived fields are stale; call kvq_layout_init");
  return ok();
}

// Split-K partition count of a decode over the tokens of L.
int check_partitions(const kvq_layout& L, int num_partitions) {
  const int64_t max_p = (int64_t(L.T) + KVQ_GROUP - 1) / KVQ_GROUP;
  if (num_partitions < 1 || num_partitions > (max_p > 1 ? max_p : 1))
    return fail(KVQ_ERR_INVALID, "num_partitions %d must be in [1, %lld]", num_partitions, (long long)max_p);
  if (num_partitions > 65535) return fail(KVQ_ERR_UNSUPPORTED, "num_partitions %d > 65535", num_partitions);
  if (L.B > 65535 || L.Hkv > 65535) return fail(KVQ_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  return KVQ_OK;
}

// A workspace too small for the partial results: a caller's (KVQ_ERR_INVALID) or
// the library's static scratch (KVQ_ERR_UNSUPPORTED).
int workspace_short(int status, size_t have, size_t need) {
  if (status == KVQ_ERR_UNSUPPORTED)
    return fail(status,
                "the partial results need %zu bytes, more than the static scratch of %zu bytes; use "
                "kv_decode_attn with a workspace, or fewer partitions",
                need, have);
  return fail(status, "workspace has %zu bytes, %zu needed", have, need);
}

}  // namespace

// Shape, bit widths and retention policy of a layout (T is the token count or a
// stream's capacity); the derived fields are not looked at.
int kvq::check_format(const kvq_layout& l) {
  const kvq_layout* L = &l;
  if (L->B < 1 || L->Hq < 1 || L->Hkv < 1 || L->T < 1)
    return fail(KVQ_ERR_INVALID, "B, Hq, Hkv and T must be >= 1 (got %d, %d, %d, %d)", L->B, L->Hq, L->Hkv, L->T);
  if (L->Hq % L->Hkv != 0) return fail(KVQ_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", L->Hq, L->Hkv);
  if (!valid_gqa(L->Hq / L->Hkv))
    return fail(KVQ_ERR_UNSUPPORTED, "Hq/Hkv = %d; supported group sizes are 1, 2, 4, 8, 16", L->Hq / L->Hkv);
  if (L->Dk < KVQ_GROUP || L->Dk % KVQ_GROUP || L->Dv < KVQ_GROUP || L->Dv % KVQ_GROUP)
    return fail(KVQ_ERR_INVALID, "Dk (%d) and Dv (%d) must be positive multiples of 32", L->Dk, L->Dv);
  if (L->Dk > KVQ_MAX_HEAD_DIM || L->Dv > KVQ_MAX_HEAD_DIM)
    return fail(KVQ_ERR_UNSUPPORTED, "Dk (%d) and Dv (%d) must be <= %d", L->Dk, L->Dv, KVQ_MAX_HEAD_DIM);
  if (!valid_bits(L->k_bits) || !valid_bits(L->v_bits))
    return fail(KVQ_ERR_UNSUPPORTED, "k_bits (%d) and v_bits (%d) must be 1, 2, 3, 4 or 8", L->k_bits, L->v_bits);
  if (L->n_recent < 0 || L->n_recent > L->T)
    return fail(KVQ_ERR_INVALID, "n_recent (%d) must be in [0, T=%d]", L->n_recent, L->T);
  if (L->log_window < 0) return fail(KVQ_ERR_INVALID, "log_window (%d) must be >= 0", L->log_window);
  if (L->k_group != 32 && L->k_group != 64 && L->k_group != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "k_group (%d) must be 32, 64 or 128", L->k_group);
  if ((L->v_group != 32 && L->v_group != 64 && L->v_group != 128) || L->Dv % L->v_group)
    return fail(KVQ_ERR_UNSUPPORTED, "v_group (%d) must be 32, 64 or 128 and divide Dv (%d)", L->v_group, L->Dv);
  if (L->flags & ~int32_t(KVQ_KEY_ROTATION)) return fail(KVQ_ERR_INVALID, "unknown layout flags 0x%x", L->flags);
  if ((L->flags & KVQ_KEY_ROTATION) && (L->Dk & (L->Dk - 1)))
    return fail(KVQ_ERR_UNSUPPORTED, "key rotation needs a power-of-two Dk (got %d)", L->Dk);
  return ok();
}

namespace {

using kvq::check_cache_ptr;
using kvq::valid_dtype;

}  // namespace

int kvq::check_cache_ptr(const void* p, const char* name) {
  if (!p) return fail(KVQ_ERR_INVALID, "cache buffer %s is NULL", name);
  if (!aligned16(p)) return fail(KVQ_ERR_INVALID, "cache buffer %s is not 16-byte aligned", name);
  return KVQ_OK;
}

// Checks and launches of a decode over a cache whose layout fields (R, Tq,
// n_groups) give the token counts and g_stride / r_stride the slab strides.
int kvq::decode_view(const kvq_layout& L, int64_t g_stride, int64_t r_stride, const void* q, int q_dtype,
                     const kvq_cache* cache, float softmax_scale, int num_partitions, void* workspace,
                     size_t workspace_bytes, float* out, void* stream, void* event_after_decode,
                     const DecodeArgs* side, int workspace_short_status, void* kernel_start,
                     void* kernel_stop) {
  int st;
  if (!cache) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (!valid_dtype(q_dtype)) return fail(KVQ_ERR_INVALID, "q_dtype %d is not KVQ_F32/F16/BF16", q_dtype);
  if (!q || !out) return fail(KVQ_ERR_INVALID, "q or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(KVQ_ERR_INVALID, "q and out must be 16-byte aligned");
  if (!std::isfinite(softmax_scale)) return fail(KVQ_ERR_INVALID, "softmax_scale is not finite");
  if ((st = check_partitions(L, num_partitions))) return st;
  if (L.n_groups > 0) {
    if ((st = check_cache_ptr(cache->k_codes, "k_codes")) || (st = check_cache_ptr(cache->k_scale, "k_scale")) ||
        (st = check_cache_ptr(cache->k_zero, "k_zero")) || (st = check_cache_ptr(cache->v_codes, "v_codes")) ||
        (st = check_cache_ptr(cache->v_scale, "v_scale")) || (st = check_cache_ptr(cache->v_zero, "v_zero")))
      return st;
  }
  if (L.R > 0) {
    if ((st = check_cache_ptr(cache->k_fp16, "k_fp16")) || (st = check_cache_ptr(cache->v_fp16, "v_fp16")))
      return st;
  }
  // Partial rows: at least P per query head whenever P > 1 (the exact count comes
  // from the plan, which needs the device), so these checks need no HIP call.
  if (num_partitions > 1) {
    const size_t least = size_t(L.B) * size_t(L.Hq) * size_t(num_partitions) * size_t(L.Dv + 4) * sizeof(float);
    if (!workspace) return fail(KVQ_ERR_INVALID, "workspace is NULL but at least %zu bytes are needed", least);
    if (!aligned16(workspace)) return fail(KVQ_ERR_INVALID, "workspace is not 16-byte aligned");
    if (workspace_bytes < least) return workspace_short(workspace_short_status, workspace_bytes, least);
  }
  kvq::DecodeArgs a{};
  a.L = L;
  a.q = q;
  a.q_dtype = q_dtype;
  a.cache = *cache;
  a.scale = softmax_scale;
  a.P = num_partitions;
  a.g_stride = g_stride;
  a.r_stride = r_stride;
  a.out = out;
  a.kernel_start = static_cast<hipEvent_t>(kernel_start);
  a.kernel_stop = static_cast<hipEvent_t>(kernel_stop);
  if (side) {
    a.side_u = side->side_u;
    a.side_codes = side->side_codes;
    a.side_scale = side->side_scale;
    a.side_zero = side->side_zero;
    a.side_rank = side->side_rank;
  }
  kvq::DecodePlan plan{};
  hipError_t e = kvq::plan_decode(a, &plan);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode planning failed: %s", hipGetErrorString(e));
  const size_t need = kvq::plan_partial_bytes(L, plan);
  if (need > 0) {
    if (workspace_bytes < need) return workspace_short(workspace_short_status, workspace_bytes, need);
    a.partials = static_cast<float*>(workspace);
  }
  e = kvq::launch_decode(a, plan, static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(event_after_decode));
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Checks and launch of a pack into a cache with slab strides g_stride / r_stride
// (L is a checked layout of the tokens [0, L.T)).
int kvq::pack_view(const kvq_layout& Lr, int64_t g_stride, int64_t r_stride, int64_t t_begin, int64_t t_count,
                   const void* K, const void* V, int kv_dtype, const kvq_cache* cache, void* stream) {
  const kvq_layout* L = &Lr;
  int st;
  if (!cache) return fail(KVQ_ERR_INVALID, "cache is NULL");
  if (!valid_dtype(kv_dtype)) return fail(KVQ_ERR_INVALID, "kv_dtype %d is not KVQ_F32/F16/BF16", kv_dtype);
  if (t_begin < 0 || t_count < 1 || t_begin + t_count > L->T)
    return fail(KVQ_ERR_INVALID, "chunk [%lld, %lld) is not inside [0, %d)", (long long)t_begin,
                (long long)(t_begin + t_count), L->T);
  if (!K || !V) return fail(KVQ_ERR_INVALID, "K or V is NULL");
  if (!aligned16(K) || !aligned16(V)) return fail(KVQ_ERR_INVALID, "K and V must be 16-byte aligned");
  const kvq::RetentionRule r = rule_of(*L);
  const int64_t q0 = kvq::quantized_before(r, t_begin), q1 = kvq::quantized_before(r, t_begin + t_count);
  if (q0 % L->k_group || q1 % L->k_group)
    return fail(KVQ_ERR_UNSUPPORTED,
                "chunk [%lld, %lld) splits a key group (%lld and %lld quantized tokens before its ends)",
                (long long)t_begin, (long long)(t_begin + t_count), (long long)q0, (long long)q1);
  kvq::PackArgs a{};
  a.L = *L;
  a.t_begin = t_begin;
  a.t_count = t_count;
  a.g_begin = q0 / KVQ_GROUP;
  a.n_groups_chunk = (q1 - q0) / KVQ_GROUP;
  a.r_begin = t_begin - q0;
  a.n_ret_chunk = (t_begin + t_count - q1) - a.r_begin;
  a.K = K;
  a.V = V;
  a.dtype = kv_dtype;
  a.cache = *cache;
  a.g_stride = g_stride;
  a.r_stride = r_stride;
  if (a.n_groups_chunk > 0) {
    if ((st = check_cache_ptr(cache->k_codes, "k_codes")) || (st = check_cache_ptr(cache->k_scale, "k_scale")) ||
        (st = check_cache_ptr(cache->k_zero, "k_zero")) || (st = check_cache_ptr(cache->v_codes, "v_codes")) ||
        (st = check_cache_ptr(cache->v_scale, "v_scale")) || (st = check_cache_ptr(cache->v_zero, "v_zero")))
      return st;
  }
  if (a.n_ret_chunk > 0) {
    if ((st = check_cache_ptr(cache->k_fp16, "k_fp16")) || (st = check_cache_ptr(cache->v_fp16, "v_fp16")))
      return st;
  }
  const hipError_t e = kvq::launch_pack(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "pack launch failed: %s", hipGetErrorString(e));
  return ok();
}

extern "C" {

int kvq_layout_init(kvq_layout* L, int B, int Hq, int Hkv, int Dk, int Dv, int T, int k_bits, int v_bits,
                    int n_recent, int log_window) {
  return kvq_layout_init_ex(L, B, Hq, Hkv, Dk, Dv, T, k_bits, v_bits, n_recent, log_window, KVQ_GROUP, KVQ_GROUP);
}

int kvq_layout_init_ex(kvq_layout* L, int B, int Hq, int Hkv, int Dk, int Dv, int T, int k_bits, int v_bits,
                       int n_recent, int log_window, int k_group, int v_group) {
  if (!L) return fail(KVQ_ERR_INVALID, "layout is NULL");
  kvq_layout l{};
  l.B = B;
  l.Hq = Hq;
  l.Hkv = Hkv;
  l.Dk = Dk;
  l.Dv = Dv;
  l.T = T;
  l.k_bits = k_bits;
  l.v_bits = v_bits;
  l.n_recent = n_recent;
  l.log_window = log_window;
  l.k_group = k_group;
  l.v_group = v_group;
  if (T >= 1 && n_recent >= 0 && n_recent <= T && log_window >= 0) {
    const int64_t R = kvq::retained_before(rule_of(l), T);
    l.R = int32_t(R);
    l.Tq = int32_t(T - R);
    l.n_groups = l.Tq / KVQ_GROUP;
  }
  const int st = check_layout(&l);
  if (st != KVQ_OK) return st;
  *L = l;
  return ok();
}

int kvq_layout_set_flags(kvq_layout* L, int flags) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  kvq_layout l = *L;
  l.flags = flags;
  if ((st = kvq::check_format(l)) != KVQ_OK) return st;
  *L = l;
  return ok();
}

int kvq_cache_sizes(const kvq_layout* L, size_t bytes_out[KVQ_NUM_CACHE_BUFFERS]) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (!bytes_out) return fail(KVQ_ERR_INVALID, "bytes_out is NULL");
  const size_t slabs = size_t(L->B) * size_t(L->Hkv);
  const size_t Tq = size_t(L->Tq), nG = size_t(L->n_groups), R = size_t(L->R);
  bytes_out[0] = slabs * Tq * size_t(L->Dk * L->k_bits / 32) * 4;   // k_codes
  bytes_out[1] = slabs * (Tq / size_t(L->k_group)) * size_t(L->Dk) * 2;  // k_scale
  bytes_out[2] = bytes_out[1];                                      // k_zero
  bytes_out[3] = slabs * Tq * size_t(L->Dv * L->v_bits / 32) * 4;   // v_codes
  bytes_out[4] = slabs * Tq * size_t(L->Dv / L->v_group) * 2;       // v_scale
  bytes_out[5] = bytes_out[4];                                      // v_zero
  bytes_out[6] = slabs * R * size_t(L->Dk) * 2;                     // k_fp16
  bytes_out[7] = slabs * R * size_t(L->Dv) * 2;                     // v_fp16
  return ok();
}

int kvq_retained_positions(const kvq_layout* L, int32_t* out, int32_t capacity) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (capacity < L->R) return fail(KVQ_ERR_INVALID, "capacity %d < R = %d", capacity, L->R);
  if (L->R > 0 && !out) return fail(KVQ_ERR_INVALID, "out is NULL");
  const kvq::RetentionRule r = rule_of(*L);
  int32_t n = 0;
  // walk positions once; a position is retained when the running count steps
  int64_t before = 0;
  for (int64_t p = 0; p < L->T; ++p) {
    const int64_t after = kvq::retained_before(r, p + 1);
    if (after != before) out[n++] = int32_t(p);
    before = after;
  }
  return ok();
}

int64_t kvq_quantized_before(const kvq_layout* L, int64_t t) {
  if (check_layout(L) != KVQ_OK) return -1;
  if (t < 0) t = 0;
  if (t > L->T) t = L->T;
  return kvq::quantized_before(rule_of(*L), t);
}

size_t kvq_decode_workspace_bytes(const kvq_layout* L, int num_partitions) {
  if (check_layout(L) != KVQ_OK || num_partitions < 1) return 0;
  if (num_partitions == 1) return 0;
  return kvq::ws_partial_bytes(*L, num_partitions);
}

int kv_quant_pack(const kvq_layout* L, int64_t t_begin, int64_t t_count, const void* K, const void* V,
                  int kv_dtype, const kvq_cache* cache, void* stream) {
  const int st = check_layout(L);
  if (st != KVQ_OK) return st;
  return kvq::pack_view(*L, L->n_groups, L->R, t_begin, t_count, K, V, kv_dtype, cache, stream);
}

int kv_decode_attn(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache, float softmax_scale,
                   int num_partitions, void* workspace, size_t workspace_bytes, float* out, void* stream) {
  return kv_decode_attn_ex(L, q, q_dtype, cache, softmax_scale, num_partitions, workspace, workspace_bytes, out,
                           stream, nullptr);
}

int kv_decode_attn_ex(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache, float softmax_scale,
                      int num_partitions, void* workspace, size_t workspace_bytes, float* out, void* stream,
                      void* event_after_decode) {
  const int st = check_layout(L);
  if (st != KVQ_OK) return st;
  return kvq::decode_view(*L, L->n_groups, L->R, q, q_dtype, cache, softmax_scale, num_partitions, workspace,
                          workspace_bytes, out, stream, event_after_decode);
}

int kv_decode_attn_timed(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache,
                         float softmax_scale, int num_partitions, void* workspace, size_t workspace_bytes,
                         float* out, void* stream, void* kernel_start, void* kernel_stop) {
  const int st = check_layout(L);
  if (st != KVQ_OK) return st;
  return kvq::decode_view(*L, L->n_groups, L->R, q, q_dtype, cache, softmax_scale, num_partitions, workspace,
                          workspace_bytes, out, stream, nullptr, nullptr, KVQ_ERR_INVALID, kernel_start,
                          kernel_stop);
}

int kv_decode_attn_noalloc(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache,
                           float softmax_scale, int num_partitions, float* out, void* stream) {
  const int st = check_layout(L);
  if (st != KVQ_OK) return st;
  void* scratch = nullptr;
  const hipError_t e = kvq::static_scratch(&scratch);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
  return kvq::decode_view(*L, L->n_groups, L->R, q, q_dtype, cache, softmax_scale, num_partitions, scratch,
                          KVQ_STATIC_SCRATCH_BYTES, out, stream, nullptr, nullptr, KVQ_ERR_UNSUPPORTED);
}

int kvq_decode_plan(const kvq_layout* L, int num_partitions, int with_side_code, kvq_decode_info* info) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (!info) return fail(KVQ_ERR_INVALID, "info is NULL");
  if ((st = check_partitions(*L, num_partitions))) return st;
  kvq::DecodeArgs a{};
  a.L = *L;
  a.P = num_partitions;
  a.side_rank = with_side_code ? 1 : 0;
  kvq::DecodePlan p{};
  const hipError_t e = kvq::plan_decode(a, &p);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode planning failed: %s", hipGetErrorString(e));
  info->kernel = p.kernel;
  info->units = p.units;
  info->ring_depth = p.depth;
  info->waves_per_simd = p.ranks;
  info->waves = p.waves;
  return ok();
}

// ------------------------------------------------------------ HeadQ side code
namespace {
int check_side(const kvq_layout* L, int rank, const float* U, const kvq_side* side) {
  if (L->flags) return fail(KVQ_ERR_UNSUPPORTED, "HeadQ side codes take a layout without flags");
  if (rank < 1 || rank > kvq::kMaxSideRank || rank > L->Dk)
    return fail(KVQ_ERR_UNSUPPORTED, "side rank %d must be in [1, min(Dk, %d)]", rank, kvq::kMaxSideRank);
  if (!U || !side) return fail(KVQ_ERR_INVALID, "U or side is NULL");
  if (!aligned16(U)) return fail(KVQ_ERR_INVALID, "U is not 16-byte aligned");
  if (L->n_groups > 0) {
    if (!side->codes || !side->scale || !side->zero) return fail(KVQ_ERR_INVALID, "side buffers must not be NULL");
    if (!aligned16(side->codes) || !aligned16(side->scale) || !aligned16(side->zero))
      return fail(KVQ_ERR_INVALID, "side buffers must be 16-byte aligned");
  }
  return ok();
}
}  // namespace

int kvq_side_sizes(const kvq_layout* L, int rank, size_t bytes_out[3]) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if (!bytes_out) return fail(KVQ_ERR_INVALID, "bytes_out is NULL");
  if (rank < 1 || rank > kvq::kMaxSideRank || rank > L->Dk)
    return fail(KVQ_ERR_UNSUPPORTED, "side rank %d must be in [1, min(Dk, %d)]", rank, kvq::kMaxSideRank);
  const size_t toks = size_t(L->B) * L->Hkv * L->Tq;
  bytes_out[0] = toks * rank;  // codes, one byte each
  bytes_out[1] = toks * 2;     // scale
  bytes_out[2] = toks * 2;     // zero
  return ok();
}

int kv_side_pack(const kvq_layout* L, int rank, int side_bits, const float* U, const void* K, int kv_dtype,
                 const kvq_cache* cache, const kvq_side* side, void* stream) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if ((st = check_side(L, rank, U, side))) return st;
  if (side_bits != 2 && side_bits != 4 && side_bits != 8)
    return fail(KVQ_ERR_UNSUPPORTED, "side_bits %d must be 2, 4 or 8", side_bits);
  if (!valid_dtype(kv_dtype)) return fail(KVQ_ERR_INVALID, "kv_dtype %d is not KVQ_F32/F16/BF16", kv_dtype);
  if (!K || !cache) return fail(KVQ_ERR_INVALID, "K or cache is NULL");
  if (!aligned16(K)) return fail(KVQ_ERR_INVALID, "K is not 16-byte aligned");
  if (L->n_groups == 0) return ok();
  if ((st = check_cache_ptr(cache->k_codes, "k_codes")) || (st = check_cache_ptr(cache->k_scale, "k_scale")) ||
      (st = check_cache_ptr(cache->k_zero, "k_zero")))
    return st;
  if (L->B > 65535 || L->Hkv > 65535) return fail(KVQ_ERR_UNSUPPORTED, "B and Hkv must be <= 65535");
  kvq::SideArgs a{};
  a.L = *L;
  a.K = K;
  a.dtype = kv_dtype;
  a.cache = *cache;
  a.U = U;
  a.rank = rank;
  a.bits = side_bits;
  a.codes = static_cast<uint8_t*>(side->codes);
  a.scale = static_cast<uint16_t*>(side->scale);
  a.zero = static_cast<uint16_t*>(side->zero);
  const hipError_t e = kvq::launch_side_pack(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "side pack launch failed: %s", hipGetErrorString(e));
  return ok();
}

int kv_decode_attn_side(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache, int rank,
                        const float* U, const kvq_side* side, float softmax_scale, int num_partitions,
                        void* workspace, size_t workspace_bytes, float* out, void* stream) {
  int st = check_layout(L);
  if (st != KVQ_OK) return st;
  if ((st = check_side(L, rank, U, side))) return st;
  kvq::DecodeArgs s{};
  s.side_u = U;
  s.side_codes = static_cast<const uint8_t*>(side->codes);
  s.side_scale = static_cast<const uint16_t*>(side->scale);
  s.side_zero = static_cast<const uint16_t*>(side->zero);
  s.side_rank = rank;
  return kvq::decode_view(*L, L->n_groups, L->R, q, q_dtype, cache, softmax_scale, num_partitions, workspace,
                          workspace_bytes, out, stream, nullptr, &s);
}

int kvq_read_probe(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink) return fail(KVQ_ERR_INVALID, "buf or sink is NULL");
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(KVQ_ERR_INVALID, "buf must be 16-byte aligned and sink 4-byte aligned");
  const hipError_t e = kvq::launch_read_probe(buf, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "read probe launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID: return "KVQ_ERR_INVALID: invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: request outside the library's limits";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP: HIP runtime error";
    default: return "unknown kvq status";
  }
}

const char* kvq_last_error(void) { return g_last_error; }

}  // extern "C"
