/*
 * kvq.h — packed low-bit KV cache and fused single-token decode attention for
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers, sizes and enums.
 *
 * What is computed (sources are the pages' technical summaries):
 *  - Keys and values of the attention KV cache are quantized group-wise and
 *    asymmetrically with separate bit widths for keys and values ("Quantize What
 *    Counts: More for Keys, Less for Values": methodology, K4V2; group size 32 for
 *    keys, results).  Keys are quantized per channel over groups of k_group = 32
 *    (default), 64 or 128 tokens ("LogQuant: Log-Distributed 2-Bit Quantization of
 *    KV Cache", section 5, per-channel keys); values per token over groups of v_group = 32 (default),
 *    64 or 128 channels (Quantize What Counts, results, sweeps the group size).
 *  - A subset of tokens stays in fp16: the newest n_recent positions and, when
 *    log_window = W > 0, log-spaced positions further back (LogQuant section 2,
 *    log-based filtering): for j = 1, 2, ... every multiple of 2^j inside
 *    [T - W*2^j, T - W*2^(j-1)), clipped at 0.
 *  - Decode attention for one new token per sequence reads the packed cache
 *    directly: out = softmax(scale * q K^T) V over all T cached tokens, where
 *    quantized and fp16 tokens may be visited in any order (LogQuant section 4,
 *    A.V = A_P.V_P); scale defaults to 1/sqrt(Dk) ("HeadQ" section 2.1; "Thin Keys,
 *    Full Values" section 2 with Dk = d_select, which may differ from Dv).
 *
 * Quantizer (bit-exact contract, all in IEEE float32 unless stated):
 *   mn, mx = min, max of the 32 values of a group
 *   s = fp16_rne(fp32(mx - mn) / fp32(2^bits - 1)),  z = fp16_rne(mn)
 *   (a stored zero of either sign is written as +0)
 *   code = 0 if s == 0, else clamp(rint_half_even((x - float(z)) / float(s)), 0, 2^bits-1)
 *   with the correctly rounded division.  Dequantized value: code * s + z.
 *
 * Packed cache layout (all buffers caller-allocated, contiguous, row-major;
 * "slab" = one (batch b, kv head h) pair, slabs ordered b-major):
 *   Tq = T - R quantized tokens in ascending position order ("compacted" order),
 *   n_groups = Tq / 32 code groups (group g = compacted tokens 32g .. 32g+31);
 *   Tq is a multiple of k_group, and key group j = code groups j*k_group/32 .. .
 *   k_codes  uint32 [B, Hkv, Tq, Dk*k_bits/32]  word w of a row holds channel
 *            w*(32/k_bits)+k at bits [k*k_bits, (k+1)*k_bits), little-endian
 *   k_scale  fp16   [B, Hkv, Tq/k_group, Dk]  one per (key group, channel)
 *   k_zero   fp16   [B, Hkv, Tq/k_group, Dk]
 *   v_codes  uint32 [B, Hkv, n_groups, Dv*v_bits]  the codes of one key group
 *            form a little-endian bit stream (bit i is bit i%32 of word i/32).
 *            With vb = v_bits, TPW = 16/vb, F = Dv*vb/8, the code of compacted
 *            token 32g + 8o + j (0 <= j < 8) and channel c = 16t + n (0 <= n < 16)
 *            sits at bit
 *              ((16o + n)*4 + j%4)*F + (t/TPW)*32 + (j/4)*r*vb + (t%TPW)*vb,
 *            r = min(TPW, Dv/16 - (t/TPW)*TPW).  When Dv*vb is a multiple of 256
 *            each 32-bit word holds, for one (o, n, j%4), the codes of TPW tiles
 *            of token j%4 in its low half and of token j%4 + 4 in its high half.
 *   v_scale  fp16   [B, Hkv, n_groups, Dv/v_group, 32]  one per token and
 *            v_group-channel group; the 32 tokens of a group are contiguous
 *   v_zero   fp16   [B, Hkv, n_groups, Dv/v_group, 32]
 *   k_fp16   fp16   [B, Hkv, R, Dk]   retained positions, ascending
 *   v_fp16   fp16   [B, Hkv, R, Dv]
 *   3-bit codes (32 is not a multiple of 3; the bit sweep of Quantize What Counts,
 *   results) use plain little-endian bit streams instead, and a code may straddle
 *   two words: key row bits [3c, 3c+3) hold channel c, and the value stream of a
 *   group holds compacted token 32g + tau, channel c at bits 3*(tau*Dv + c) .. +3.
 *
 * Threading and ownership: the library allocates no device memory, keeps no
 * state between calls (apart from the thread-local last-error text), never
 * synchronizes, and enqueues work only on the stream it is given.  Every pointer
 * stays owned by the caller and must stay valid until the enqueued work is done.
 *
 * Errors: every call validates its arguments on the host before launching
 * anything and returns KVQ_ERR_INVALID / KVQ_ERR_UNSUPPORTED without touching the
 * GPU; a failed launch returns KVQ_ERR_HIP.  kvq_last_error() gives the reason.
 * Unchecked preconditions: inputs are finite, |values| and group ranges stay
 * inside the fp16 range, buffers have the sizes kvq_cache_sizes() reports, and
 * device pointers are 16-byte aligned device memory.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = 1,      /* bad argument (null pointer, out-of-range value, misalignment) */
  KVQ_ERR_UNSUPPORTED = 2,  /* valid request the library does not handle (see limits below) */
  KVQ_ERR_HIP = 3           /* a HIP runtime call or kernel launch failed */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 } kvq_dtype;

enum { KVQ_GROUP = 32, KVQ_MAX_HEAD_DIM = 256, KVQ_MAX_GQA = 16, KVQ_NUM_CACHE_BUFFERS = 8 };

/* Shape and policy of one packed cache.  Fill with kvq_layout_init(); treat as
 * read-only afterwards (calls re-derive and check R, Tq, n_groups). */
typedef struct {
  int32_t B, Hq, Hkv, Dk, Dv, T;
  int32_t k_bits, v_bits;         /* each in {1, 2, 3, 4, 8} (1- and 3-bit caches decode on the vector-ALU kernel) */
  int32_t n_recent;               /* newest positions kept in fp16 (0..T; T = no quantization) */
  int32_t log_window;             /* W of the log-spaced fp16 positions; 0 = none */
  int32_t k_group;                /* tokens per key group: 32, 64 or 128 (Tq a multiple of it) */
  int32_t v_group;                /* channels per value group: 32, 64 or 128, dividing Dv */
  int32_t R, Tq, n_groups;        /* derived: retained count, quantized count, Tq / 32 */
  int32_t flags;                  /* KVQ_KEY_ROTATION or 0 (kvq_layout_set_flags) */
} kvq_layout;

/* Device pointers of the eight cache buffers described above.  Buffers a call
 * does not touch may be NULL (e.g. k_fp16 / v_fp16 when R == 0). */
typedef struct {
  void *k_codes, *k_scale, *k_zero;
  void *v_codes, *v_scale, *v_zero;
  void *k_fp16, *v_fp16;
} kvq_cache;

/* Fill *L and derive R, Tq, n_groups.  Limits (else KVQ_ERR_INVALID, or
 * KVQ_ERR_UNSUPPORTED where the request is well-formed): all sizes >= 1,
 * Hq % Hkv == 0 with Hq / Hkv <= KVQ_MAX_GQA, Dk and Dv multiples of 32 up to
 * KVQ_MAX_HEAD_DIM, bits in {1, 2, 3, 4, 8}, 0 <= n_recent <= T, log_window >= 0, and
 * the quantized token count Tq a multiple of 32 (choose n_recent accordingly). */
int kvq_layout_init(kvq_layout* L, int B, int Hq, int Hkv, int Dk, int Dv, int T,
                    int k_bits, int v_bits, int n_recent, int log_window);

/* kvq_layout_init with keys in groups of k_group tokens (32, 64 or 128; the quantized
 * count Tq must be a multiple of it) and values in groups of v_group channels (32, 64
 * or 128, dividing Dv); KVQ_ERR_UNSUPPORTED otherwise.  kvq_layout_init is this with
 * k_group = v_group = 32. */
int kvq_layout_init_ex(kvq_layout* L, int B, int Hq, int Hkv, int Dk, int Dv, int T,
                       int k_bits, int v_bits, int n_recent, int log_window, int k_group, int v_group);

/* Key-only rotation ("Quantize What Counts", technical summary: contributions,
 * orthogonality and integration; results, rotation integration: rotating only the
 * keys before they are quantized spreads outlier channels over all channels).
 * With KVQ_KEY_ROTATION every key row k (quantized or kept in fp16) is replaced by
 * H k before it is stored, H the orthonormal Walsh-Hadamard transform of width Dk
 * in Sylvester order, computed in float32 as butterflies for h = 1, 2, 4, ..., Dk/2
 * (entries j and j + h of every 2h-block become a + b and a - b, in that order)
 * followed by one multiply with float32(2^(-m/2)), Dk = 2^m (for odd m,
 * float32(sqrt(1/2)) * 2^(-(m-1)/2)); decode applies the same H to the query, so
 * scores are unchanged in exact arithmetic.  The packed cache then holds the
 * rotated keys; a cache must be decoded with the flags it was packed with. */
enum { KVQ_KEY_ROTATION = 1 };

/* Set the flags of a layout filled by kvq_layout_init(_ex): 0 or KVQ_KEY_ROTATION
 * (KVQ_ERR_INVALID for other bits; KVQ_ERR_UNSUPPORTED for rotation unless Dk is a
 * power of two).  Streams take their flags from kvq_stream_set_flags; HeadQ side
 * codes take a layout without flags. */
int kvq_layout_set_flags(kvq_layout* L, int flags);

/* Byte sizes of the eight kvq_cache buffers, in kvq_cache field order. */
int kvq_cache_sizes(const kvq_layout* L, size_t bytes_out[KVQ_NUM_CACHE_BUFFERS]);

/* Host-side list of the R retained positions (ascending) into out[0..capacity).
 * Returns KVQ_ERR_INVALID if capacity < R.  No GPU work. */
int kvq_retained_positions(const kvq_layout* L, int32_t* out, int32_t capacity);

/* Number of quantized (non-retained) positions in [0, t).  Host-side, no GPU work;
 * a chunk [t0, t1) can be packed on its own when both counts are multiples of 32. */
int64_t kvq_quantized_before(const kvq_layout* L, int64_t t);

/* Workspace kv_decode_attn needs for num_partitions sequence partitions (0 when
 * num_partitions == 1): B*Hq*4*num_partitions*(Dv+4) floats of partial results
 * (the decode kernel may cut the key groups into up to 4*num_partitions runs).
 * Returns 0 for an invalid layout. */
size_t kvq_decode_workspace_bytes(const kvq_layout* L, int num_partitions);

/*
 * kv_quant_pack — quantize and pack positions [t_begin, t_begin + t_count) of the
 * cache described by L (the whole cache: t_begin = 0, t_count = T).
 *   K: [B, Hkv, t_count, Dk], V: [B, Hkv, t_count, Dv] device arrays of dtype
 *      kv_dtype (KVQ_F32 / KVQ_F16 / KVQ_BF16), contiguous; row j is position
 *      t_begin + j.
 *   cache: buffers for the WHOLE cache; the call writes the key groups, value rows
 *      and fp16 rows that belong to the chunk and nothing else, so chunks can be
 *      packed independently (e.g. a prefill chunk appended to an existing cache).
 *   stream: hipStream_t to enqueue on (NULL = default stream).
 * The number of quantized positions before t_begin and before t_begin + t_count
 * must both be multiples of k_group (else KVQ_ERR_UNSUPPORTED).  Output is
 * deterministic: codes, scales and zeros follow the quantizer contract above bit
 * for bit.
 */
int kv_quant_pack(const kvq_layout* L, int64_t t_begin, int64_t t_count,
                  const void* K, const void* V, int kv_dtype,
                  const kvq_cache* cache, void* stream);

/*
 * kv_decode_attn — single-token decode attention over a packed cache: one decode
 * kernel whose waves each take a contiguous run of key groups of one (batch row,
 * kv head) pair and, when P > 1, one merge kernel after it on the same stream.
 *   q:   [B, Hq, Dk] device array of dtype q_dtype; query head i reads KV head
 *        i / (Hq / Hkv) (grouped-query attention: the Hq/Hkv queries of one KV head
 *        share each read of its cache).
 *   softmax_scale: scale of the scores (finite; pass 1/sqrtf(Dk) for the usual one).
 *   num_partitions: P, the split-K factor: the key groups of every (batch row, kv
 *        head) pair are cut into P contiguous runs processed in parallel, each with
 *        a share of the retained tokens, and the partial results are merged.  The
 *        library chooses the run boundaries: near-equal (integer division) for the
 *        vector-ALU kernel; for the matrix-core kernel the P runs may be cut further
 *        into 2P, 4P or 8P and sized by dispatch order (within about +-20% of equal).
 *        Results differ only in rounding.  1 <= P <= max(1, ceil(T/32)).
 *   workspace / workspace_bytes: 16-byte aligned device memory for the partial
 *        results: kvq_decode_workspace_bytes(L, P) bytes always suffice (the exact
 *        need is B * Hq * units * (Dv + 4) floats, units from kvq_decode_plan; 0
 *        when units == 1, and then workspace may be NULL); no initialisation needed.  A workspace serves one call at a time: calls that
 *        overlap on the GPU (different streams) need separate workspaces.
 *   out: [B, Hq, Dv] float32 device array.
 * Partial results of the partitions are merged on the device.
 */
int kv_decode_attn(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache,
                   float softmax_scale, int num_partitions, void* workspace,
                   size_t workspace_bytes, float* out, void* stream);

/*
 * kv_decode_attn_ex — kv_decode_attn with a timing hook for callers that measure
 * the two kernels separately.  event_after_decode: a hipEvent_t created by the
 * caller (NULL = none, then identical to kv_decode_attn); it is recorded on
 * `stream` right after the decode kernel is enqueued and before the merge kernel
 * (when P == 1 there is no merge and it is recorded after the only kernel).  A
 * failed record returns KVQ_ERR_HIP.  All other arguments as kv_decode_attn.
 */
int kv_decode_attn_ex(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache,
                      float softmax_scale, int num_partitions, void* workspace, size_t workspace_bytes,
                      float* out, void* stream, void* event_after_decode);

/*
 * kv_decode_attn_timed — kv_decode_attn for callers that time the decode kernel
 * alone (the work unit whose bytes the decode's roofline counts).  kernel_start,
 * kernel_stop: hipEvent_t handles created by the caller (either may be NULL, both
 * NULL = kv_decode_attn).  The decode kernel is launched with hipExtLaunchKernel
 * with them as its start and stop events (the runtime's timing of that one kernel
 * command, which leaves out the host's launch time); the merge kernel (when P > 1)
 * follows untimed.  A failed launch returns KVQ_ERR_HIP.  All other
 * arguments, results and errors as kv_decode_attn.
 */
int kv_decode_attn_timed(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache,
                         float softmax_scale, int num_partitions, void* workspace, size_t workspace_bytes,
                         float* out, void* stream, void* kernel_start, void* kernel_stop);

/*
 * kv_decode_attn_noalloc — kv_decode_attn for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, and the same kernels.
 * The partial results go to a static device array of KVQ_STATIC_SCRATCH_BYTES
 * (16 MiB) that each GPU the library runs on holds until the process ends; the call
 * allocates nothing.  A request whose partial results exceed it (B * Hq * units *
 * (Dv + 4) floats, units from kvq_decode_plan; nothing when units == 1) returns
 * KVQ_ERR_UNSUPPORTED before any launch.  Every call on one GPU shares that GPU's
 * array: calls that overlap on the GPU (other streams, other threads) race and
 * give wrong results; calls enqueued on one stream are ordered and safe.
 */
enum { KVQ_STATIC_SCRATCH_BYTES = 16 << 20 };
int kv_decode_attn_noalloc(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache,
                           float softmax_scale, int num_partitions, float* out, void* stream);

/*
 * kvq_decode_plan — which decode kernel kv_decode_attn (with_side_code = 0) or
 * kv_decode_attn_side (with_side_code != 0) runs for this layout and partition
 * count on the calling thread's current device, and how it cuts the work.  No GPU
 * work is enqueued; the device's compute-unit count is read (once per device).
 *   kernel: KVQ_KERNEL_MFMA, the matrix-core kernel, for 4 query heads per KV head,
 *     Dv = 128, Dk in {32, 64, 128} and 2/4/8-bit codes with Dk * k_bits >= 128, no
 *     side code; KVQ_KERNEL_VALU, the vector-ALU kernel, for every other layout.  A
 *     layout the matrix-core kernel takes never runs on the other one: a failure
 *     there is returned as KVQ_ERR_HIP.
 *   units: partial results per query head that the merge kernel folds (1: the
 *     decode kernel writes the output and no merge runs).
 *   ring_depth: key groups each wave of the matrix-core kernel keeps in its LDS
 *     ring (2 or 3); waves_per_simd: waves of that grid per SIMD; both 0 for the
 *     vector-ALU kernel.  waves: waves the decode kernel launches.
 * Errors: as kv_decode_attn for the layout and num_partitions; KVQ_ERR_HIP if the
 * device cannot be queried.
 */
enum { KVQ_KERNEL_MFMA = 1, KVQ_KERNEL_VALU = 2 };
typedef struct {
  int32_t kernel;
  int32_t units;
  int32_t ring_depth;
  int32_t waves_per_simd;
  int64_t waves;
} kvq_decode_info;
int kvq_decode_plan(const kvq_layout* L, int num_partitions, int with_side_code, kvq_decode_info* info);

/* ------------------------------------------------------------------ streaming
 *
 * A streaming cache grows by one decode-time token per kv_stream_append call
 * (LogQuant technical summary, section 2, dynamic adjustment: as tokens arrive the
 * fp16 density of the older windows halves, so tokens leave the fp16 set at
 * regular intervals; section 4: the cached tokens may be stored in any order).
 *  - Retention at t tokens is the rule above with T = t.  Positions are absolute,
 *    so a token that has left the fp16 set never re-enters it; this needs
 *    log_window == 0 or n_recent >= log_window.
 *  - An appended token is stored in fp16 (round to nearest even).
 *  - A token that leaves the fp16 set becomes pending: it stays in its fp16 row and
 *    is attended as fp16 until 32 tokens are pending.  Then the 32 pending tokens
 *    of lowest position, in ascending position, are quantized from their fp16
 *    values as the next key group (the quantizer contract and group format above)
 *    and their rows are freed.  The rows in use are always [0, n_rows): rows past
 *    the new end move into the freed ones.
 *  - Decode attends over the n_groups packed groups and the n_rows fp16 rows.
 * Buffers: the eight kvq_cache buffers with g_cap groups and r_cap rows per slab
 * (slab strides; only the first n_groups / n_rows are meaningful):
 *   k_codes uint32 [B, Hkv, 32*g_cap, Dk*k_bits/32]   (32 rows per group)
 *   k_scale, k_zero fp16 [B, Hkv, g_cap, Dk]
 *   v_codes uint32 [B, Hkv, g_cap, Dv*v_bits]
 *   v_scale, v_zero fp16 [B, Hkv, g_cap, Dv/v_group, 32]
 *   k_fp16 fp16 [B, Hkv, r_cap, Dk], v_fp16 fp16 [B, Hkv, r_cap, Dv]
 * The host state (kvq_stream, caller-owned) advances when a call is enqueued, so
 * all calls on one stream state must be enqueued in order on one HIP stream.  A
 * call that fails leaves the state as it was.
 */
enum { KVQ_STREAM_MAX_ROWS = 4096 };

typedef struct {
  kvq_layout L;        /* format: B, Hq, Hkv, Dk, Dv, bits, n_recent, log_window;
                          L.T = capacity (most tokens the stream may hold);
                          L.R, L.Tq, L.n_groups are unused (0) */
  int32_t t;           /* tokens in the stream (positions 0 .. t-1) */
  int32_t n_groups;    /* key groups packed, per slab */
  int32_t n_rows;      /* fp16 rows in use, per slab */
  int32_t n_pending;   /* rows among them whose token has left the fp16 set */
  int32_t g_cap;       /* group capacity per slab: capacity / 32 */
  int32_t r_cap;       /* fp16 row capacity per slab (a bound on n_rows over the
                          stream's life, at most KVQ_STREAM_MAX_ROWS) */
  int32_t row_pos[KVQ_STREAM_MAX_ROWS];      /* position of the token in row i < n_rows */
  uint8_t row_pending[KVQ_STREAM_MAX_ROWS];  /* 1 if row i's token is pending */
} kvq_stream;

/* What one appended token changes on the device (filled by kvq_stream_plan). */
typedef struct {
  int32_t new_row;           /* fp16 row the token is written to */
  int32_t group;             /* index of the key group formed, or -1 */
  int32_t member_rows[32];   /* rows of the group's tokens (before the moves), ascending position */
  int32_t member_pos[32];    /* their positions */
  int32_t n_moves;           /* rows moved into freed rows once the group is packed */
  int32_t move_src[32], move_dst[32];
} kvq_stream_step;

/* Start an empty stream (t = 0) for at most `capacity` tokens.  Limits as
 * kvq_layout_init (without its multiple-of-32 rule), plus: log_window == 0 or
 * n_recent >= log_window (KVQ_ERR_UNSUPPORTED otherwise), capacity >= 1, and an fp16
 * row bound of at most KVQ_STREAM_MAX_ROWS (KVQ_ERR_UNSUPPORTED otherwise). */
int kvq_stream_init(kvq_stream* S, int B, int Hq, int Hkv, int Dk, int Dv, int capacity,
                    int k_bits, int v_bits, int n_recent, int log_window);

/* kvq_stream_init with values in groups of v_group channels (as kvq_layout_init_ex).
 * Stream key groups are 32 tokens (a group forms from 32 pending tokens). */
int kvq_stream_init_ex(kvq_stream* S, int B, int Hq, int Hkv, int Dk, int Dv, int capacity,
                       int k_bits, int v_bits, int n_recent, int log_window, int v_group);

/* Set the layout flags of an empty stream (t == 0, else KVQ_ERR_INVALID), as
 * kvq_layout_set_flags: with KVQ_KEY_ROTATION prefill packs rotated keys, append
 * rotates each new key row in float32 before its fp16 rounding (so groups form from
 * rotated rows), and decode rotates the query. */
int kvq_stream_set_flags(kvq_stream* S, int flags);

/* Byte sizes of the eight buffers of a stream's cache, in kvq_cache field order. */
int kvq_stream_cache_sizes(const kvq_stream* S, size_t bytes_out[KVQ_NUM_CACHE_BUFFERS]);

/* Workspace kv_stream_decode needs for num_partitions (as kvq_decode_workspace_bytes). */
size_t kvq_stream_workspace_bytes(const kvq_stream* S, int num_partitions);

/* Host-side bookkeeping of one append, no GPU work: advances *S by one token and
 * describes in *step what the device must do.  kv_stream_append calls it; it is
 * exported so that the bookkeeping can be inspected and tested on its own.
 * KVQ_ERR_INVALID if the stream is full (t == capacity). */
int kvq_stream_plan(kvq_stream* S, kvq_stream_step* step);

/* kv_stream_prefill — start an empty stream from the one-shot cache of its first
 * T0 tokens (kv_quant_pack's grouping: quantized positions in ascending order,
 * retained positions in fp16 rows in ascending order; nothing pending).
 *   K [B, Hkv, T0, Dk], V [B, Hkv, T0, Dv]: device arrays of kv_dtype.
 * Needs t == 0, 1 <= T0 <= capacity and a quantized count at T0 that is a multiple
 * of 32 (else KVQ_ERR_UNSUPPORTED). */
int kv_stream_prefill(kvq_stream* S, int T0, const void* K, const void* V, int kv_dtype,
                      const kvq_cache* cache, void* stream);

/* kv_stream_append — append the token at position t.  k_new [B, Hkv, Dk] and
 * v_new [B, Hkv, Dv]: device arrays of kv_dtype, 16-byte aligned.  One kernel
 * launch: the token's fp16 row, and when a group forms, its codes, scales and
 * zeros and the row moves.  KVQ_ERR_INVALID when the stream is full. */
int kv_stream_append(kvq_stream* S, const void* k_new, const void* v_new, int kv_dtype,
                     const kvq_cache* cache, void* stream);

/* kv_stream_decode — kv_decode_attn over the stream's t tokens (arguments as
 * there; 1 <= num_partitions <= max(1, ceil(t / 32)); needs t >= 1). */
int kv_stream_decode(const kvq_stream* S, const void* q, int q_dtype, const kvq_cache* cache,
                     float softmax_scale, int num_partitions, void* workspace, size_t workspace_bytes,
                     float* out, void* stream);

/* ---- HeadQ side code ("HeadQ", section 3, methodology): write and read mechanics.
 * Write: for every quantized token j of a packed cache, e_j = k_j - k_hat_j (k_hat_j
 * from the cache's codes, scales and zeros), y_j = U_h^T e_j (summed in float64 over
 * channels in ascending order, rounded once to float32), and the r coefficients of
 * y_j quantized as one group with side_bits bits under the quantizer contract above.
 * Read: decode adds (U_h^T q) . z_hat_j, in the scores' units, to each quantized
 * token's score; fp16-retained tokens get no correction.  U is caller-supplied
 * (the page learns it by PCA on calibration queries): float32 [Hkv, Dk, rank],
 * 1 <= rank <= min(Dk, 16).  Buffers (caller-allocated, sizes from kvq_side_sizes):
 *   codes uint8 [B, Hkv, Tq, rank] (one code per byte), scale / zero fp16 [B, Hkv, Tq].
 * Only caches packed with kvq_layout_init(_ex) (not streams).  Decode with a side
 * code runs on the vector-ALU kernel. */
typedef struct {
  void *codes, *scale, *zero;
} kvq_side;

/* Byte sizes of the three side buffers (codes, scale, zero). */
int kvq_side_sizes(const kvq_layout* L, int rank, size_t bytes_out[3]);

/* Write the side code of every quantized token.  K: the same [B, Hkv, T, Dk] keys the
 * cache was packed from (device, kv_dtype); cache: a packed cache (k_codes, k_scale,
 * k_zero are read); side_bits in {2, 4, 8}.  Enqueued on `stream`. */
int kv_side_pack(const kvq_layout* L, int rank, int side_bits, const float* U, const void* K, int kv_dtype,
                 const kvq_cache* cache, const kvq_side* side, void* stream);

/* kv_decode_attn with the HeadQ logit correction of `side` (same arguments otherwise). */
int kv_decode_attn_side(const kvq_layout* L, const void* q, int q_dtype, const kvq_cache* cache, int rank,
                        const float* U, const kvq_side* side, float softmax_scale, int num_partitions,
                        void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * kvq_read_probe — measurement support, not part of the decode path: reads
 * buf[0, bytes) once (bytes rounded down to a multiple of 16) with a grid-wide
 * streaming read of non-temporal loads (the cache policy of the decode kernel's
 * copies), so that a caller can time the HBM read rate the
 * device reaches and report it next to the decode kernel's.  buf: 16-byte
 * aligned device memory, owned by the caller.  sink: 4 bytes of device memory
 * the kernel may write (it keeps the reads from being optimized away; its
 * content is unspecified).  stream: hipStream_t (NULL = default).  Errors:
 * KVQ_ERR_INVALID for a NULL or misaligned pointer, KVQ_ERR_HIP for a failed
 * launch.
 */
int kvq_read_probe(const void* buf, size_t bytes, void* sink, void* stream);

/* Static text for a status code. */
const char* kvq_status_string(int status);

/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
