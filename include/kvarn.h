/*
 * kvarn.h -- C ABI of the KVarN hot path on MI355X (gfx950).
 *
 * KVarN quantizes a KV cache without calibration: each 128-token group of
 * post-RoPE K and V of one KV head is rotated along the channel axis by a
 * Hadamard matrix, variance-normalized over the token and channel axes with
 * 16 Sinkhorn-style iterations, rounded to nearest and stored as a record of
 * codes plus scale metadata.  The first 128 tokens (the sink) and the
 * in-progress group (the tail) stay exact in fp16.  Decode attention reads
 * the records directly in the rotated frame and rotates its output back once.
 *
 * Sources (cited by page title and section):
 *   [P1] "KVarN: Variance-Normalized KV-Cache Quantization Mitigates Error
 *        Accumulation in Reasoning Tasks" (fig1.dev summary of arXiv
 *        2606.03458): "What it is", "Why it matters".
 *   [P2] "KVarN KV Cache: Implementation and Benchmarks" (anbeeld.com):
 *        §1 "Where KVarN Comes From", §2.1 "Sink, Body, And Tail",
 *        §5 "Changing Only The Format", §6 "Splitting K And V".
 *
 * Conventions shared by every entry point:
 *   - Every buffer is allocated and owned by the caller.  The library never
 *     allocates, frees or synchronizes; all work is queued on `stream` (a
 *     hipStream_t; NULL = the default stream) in call order.
 *   - Pointers marked "device" must be device-accessible memory of the
 *     current HIP device; "host" pointers are read before the call returns.
 *   - Argument errors are detected on the host before anything is queued and
 *     returned as a negative kvarn_status; kvarn_last_error() then holds a
 *     message (thread-local).  Launch failures return KVARN_EHIP.
 *   - fp16 = IEEE binary16.  Inputs must be finite and small enough that the
 *     scales of reading R8 below fit fp16 (|x| < 2^12 is always safe).
 *   - The record layout (reading R9 of the oracle):
 *       record = [codes][s: 128 x fp16][c: D x fp16],
 *       K codes token-major (row t = token t's D codes),
 *       V codes channel-major (row j = channel j's 128 codes);
 *       a row is a little-endian bit stream in which code i occupies bits
 *       [b*i, b*i + b) (for b = 2, 4, 8: bit b*(i mod 32/b) of 32-bit
 *       little-endian word floor(i*b/32)).  Dequantized value (rotated
 *       frame): s_t * (code_tj - (2^b-1)/2) * c_j; original frame: times
 *       H_D/sqrt(D).
 *   - Code widths b are 2, 3, 4, 5, 6 or 8 bits [P2 §5 "Changing Only The
 *     Format", §6 "Splitting K And V"], chosen for K and V independently:
 *     every ordered (k_bits, v_bits) pair of them is supported.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVARN_OK = 0,
  KVARN_EINVAL = -1,       /* null pointer, negative size, bad field */
  KVARN_EUNSUPPORTED = -2, /* valid but not implemented (head_dim, bits, GQA) */
  KVARN_ERANGE = -3,       /* a length exceeds a capacity */
  KVARN_EWORKSPACE = -4,   /* workspace too small */
  KVARN_EHIP = -5          /* the HIP runtime reported an error */
} kvarn_status;

/* Group, sink and tail capacity are 128 tokens each [P2 §2.1]. */
#define KVARN_GROUP 128
#define KVARN_SINK 128
#define KVARN_SINKHORN_ITERS 16 /* [P2 §1] */

typedef struct {
  int32_t head_dim;       /* D: 128 or 256 */
  int32_t num_q_heads;    /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;   /* Hkv; Hq/Hkv must be 1, 2 or 4 */
  int32_t k_bits;         /* 2, 3, 4, 5, 6 or 8 */
  int32_t v_bits;         /* 2, 3, 4, 5, 6 or 8 */
  int32_t group;          /* must be 128 */
  int32_t sink;           /* must be 128 */
  int32_t sinkhorn_iters; /* 0..64; KVarN uses 16 */
} kvarn_config;

/*
 * Cache view (pointers only).  Element (b, h, i, d) of an fp16 block is at
 * index ((b*Hkv + h)*128 + i)*D + d.  seq_len[b] = tokens cached for
 * request b.  Positions [0,128) live in the sink, group g covers positions
 * [128+128g, 256+128g), and the tail holds positions [128+128*G, n) with
 * G = max(0,(n-128)/128) sealed groups [P2 §2.1].  The cache holds at most
 * 128 + 128*max_groups + 127 tokens per request.
 *
 * Records.  Each (request b, KV head h, group g) owns one pair of
 * kvarn_group_bytes(cfg) bytes: the K record first, then the V record.
 *   - Contiguous (block_table NULL): pair (b*Hkv + h)*max_groups + g of
 *     `records`, which holds batch*Hkv*max_groups pairs.
 *   - Paged (block_table non-NULL): `records` is a pool of num_blocks blocks,
 *     a block being the Hkv pairs of one 128-token group, and group g of
 *     request b lives in block block_table[b*max_groups + g] (device int32
 *     [batch][max_groups]): pair block*Hkv + h.  This is the block table of
 *     a paged KV cache with 128-token blocks, which lets requests share one
 *     pool and grow without copying.  An entry outside [0, num_blocks) gives
 *     the group no storage: sealing skips it and decoding treats it as
 *     absent (an empty group), so a bad entry never addresses memory outside
 *     the pool.  Entries for groups not yet sealed are not read by decoding.
 */
typedef struct {
  void *sink_k, *sink_v; /* device fp16 [batch][Hkv][128][D] */
  void *tail_k, *tail_v; /* device fp16 [batch][Hkv][128][D] */
  void *records;         /* device record pairs (see above) */
  int32_t *seq_len;      /* device int32 [batch] */
  int32_t batch;
  int32_t max_groups;            /* groups per request (table row length when paged) */
  const int32_t *block_table;    /* NULL (contiguous) or device int32 [batch][max_groups] */
  int32_t num_blocks;            /* blocks in the pool when paged; ignored otherwise */
} kvarn_cache;

/* Pure host helpers (no GPU needed). ---------------------------------- */

/* Checks a config; KVARN_OK or the status an entry point would return. */
kvarn_status kvarn_check_config(const kvarn_config *cfg);

/* Bytes of one record: 128*D*bits/8 + 2*128 + 2*D; 0 if unsupported
 * (bits must be 2, 3, 4, 5, 6 or 8). */
size_t kvarn_record_bytes(int32_t head_dim, int32_t bits);

/* Bytes of one (K record, V record) pair; 0 for an invalid config. */
size_t kvarn_group_bytes(const kvarn_config *cfg);

/* Workspace that kvarn_decode_attn needs for this batch and max_groups. */
size_t kvarn_decode_workspace_bytes(const kvarn_config *cfg, int32_t batch, int32_t max_groups);

/*
 * The launch plan kvarn_decode_attn uses for this configuration, batch and
 * max_groups on the current device (a device-free plan if there is none):
 * out (host int32 [5]) = {record splits per (request, KV head), exact splits
 * per (request, KV head), groups per wave at most, record workgroups, exact
 * workgroups}.  The plan depends on the capacity (max_groups), not on the
 * lengths, so every call on one cache launches the same grid.
 */
kvarn_status kvarn_decode_plan(const kvarn_config *cfg, int32_t batch, int32_t max_groups, int32_t *out);

/* Message of the last error on this thread ("" if none). */
const char *kvarn_last_error(void);

/* Stable name of a status code. */
const char *kvarn_status_string(kvarn_status s);

/* Hot-path entry points. ------------------------------------------------ */

/*
 * Append one token per request [P2 §2.1].  k_new, v_new: device fp16
 * [batch][Hkv][D], post-RoPE.  For each request b with n = seq_len[b], the
 * token goes to sink[n] if n < 128, else to tail[(n-128) mod 128]; then
 * seq_len[b] = n+1.  A request whose cache is full (n >= 128 +
 * 128*max_groups + 127, so the token would complete a group that has no
 * record slot) is left unchanged.  Call kvarn_seal_group after every append
 * so a full tail is sealed before the next append overwrites it.  Between
 * the two calls, do not decode: decoding counts a group as sealed as soon as
 * seq_len covers it, so it would read that group's record before it is
 * written (and no longer read the tail).  kvarn_append_seal does both in one
 * launch and has no such window.
 */
kvarn_status kvarn_append(const kvarn_config *cfg, const kvarn_cache *cache,
                          const void *k_new, const void *v_new, void *stream);

/*
 * Seal on arrival [P2 §2.1: a group is quantized the moment its last token
 * arrives].  The group sealed for request b is the one whose 128 tokens fill
 * its tail: with n = seq_len[b] (read on the device, so no host
 * synchronization is needed), the newest token completed group
 * g = (n-128)/128 - 1 when n >= 256 and (n-128) mod 128 == 0.  That group is
 * quantized from the tail into record g for every KV head, K and V: Hadamard
 * rotation, `sinkhorn_iters` alternating token and channel RMS rescalings,
 * per-token round to nearest [P1 "What it is"; P2 §1].  The tail then counts
 * as empty (no data moves).
 *
 * Two forms:
 *   - Predicate form: d_req == NULL, d_group == NULL, n == batch.  Every
 *     request whose tail just filled is sealed; the others are untouched.
 *   - List form: d_req, d_group: device int32 [n].  Entry i asks to seal
 *     group d_group[i] of request d_req[i]; it is carried out only if that
 *     group is the one whose tokens fill the request's tail (see above), and
 *     skipped otherwise (stale or future groups, requests outside
 *     [0, batch)), so a wrong list never writes a record from the wrong
 *     tokens.  Entries may come in any order; a repeated entry writes the
 *     same bytes twice.  One workgroup per entry, KV head and K|V, so a
 *     caller that knows which requests are due launches only those.
 * n == 0 (an empty list; its pointers may then be NULL) or max_groups == 0
 * queues nothing.
 */
kvarn_status kvarn_seal_group(const kvarn_config *cfg, const kvarn_cache *cache,
                              const int32_t *d_req, const int32_t *d_group, int32_t n, void *stream);

/*
 * kvarn_append followed by kvarn_seal_group, in one launch (one workgroup
 * per KV head and K|V instead of two launches per decode step) [P2 §2.1:
 * append to the tail; seal a group when its last token arrives].  Same
 * arguments and results as the two calls: the token goes to its slot, a
 * tail it completes is sealed into its record, and seq_len[b] advances by
 * one (not for a full cache).  While the launch runs, bits 23..30 of
 * seq_len[b] count the request's workgroups that have read the length (the
 * last one clears them), so nothing else may access seq_len until it
 * completes (stream order guarantees this for work on the same stream).
 * Requires num_kv_heads <= 127 (else KVARN_EUNSUPPORTED) and a capacity
 * 128 + 128*max_groups + 127 below 2^23 tokens (else KVARN_ERANGE).
 */
kvarn_status kvarn_append_seal(const kvarn_config *cfg, const kvarn_cache *cache,
                               const void *k_new, const void *v_new, void *stream);

/*
 * Bulk ingest of a prompt: for each request b, tokens [0, len_host[b]) of
 * k, v (device fp16 [batch][Hkv][src_tokens][D]) fill the sink, every
 * complete group is sealed into its record, the rest goes to the tail, and
 * seq_len[b] = len_host[b].  len_host is a host array [batch]; each length
 * must be <= src_tokens and <= the cache capacity (else KVARN_ERANGE).
 */
kvarn_status kvarn_prefill(const kvarn_config *cfg, const kvarn_cache *cache,
                           const void *k, const void *v, int64_t src_tokens,
                           const int32_t *len_host, void *stream);

/*
 * kvarn_prefill for n_layers layer caches of one model at once (the same
 * prompt lengths in every layer): one copy launch and one seal launch per 16
 * layers instead of two launches per layer, so a short prompt, whose groups
 * alone would leave most compute units idle, fills the GPU with the tiles of
 * all its layers [P2 §2.1; the sealing of P1 "What it is", P2 §1].
 * caches: host array [n_layers] of cache views sharing batch and max_groups
 * (each with its own buffers, paged or not); k, v: host arrays [n_layers] of
 * device fp16 [batch][Hkv][src_tokens][D] pointers; len_host as for
 * kvarn_prefill.  Results equal n_layers kvarn_prefill calls.
 */
kvarn_status kvarn_prefill_layers(const kvarn_config *cfg, const kvarn_cache *caches, int32_t n_layers,
                                  const void *const *k, const void *const *v, int64_t src_tokens,
                                  const int32_t *len_host, void *stream);

/*
 * Decode attention [P2 §1, §2.1]: for every request b and query head h
 * (KV head floor(h*Hkv/Hq)), attends the query q (device fp16 [batch][Hq][D],
 * post-RoPE) over all seq_len[b] cached positions: the exact sink and tail in
 * the original frame, the sealed records in the rotated frame with the query
 * rotated by the same Hadamard matrix; the record part of the output is
 * rotated back once.  out: device fp32 [batch][Hq][D].  softmax_scale
 * multiplies q.k (use 1/sqrt(D)).  workspace: device, at least
 * kvarn_decode_workspace_bytes(cfg, batch, max_groups) bytes, 256-byte
 * aligned; its contents are scratch, and calls sharing a workspace must not
 * overlap.  A request with seq_len 0 gets zeros.
 */
kvarn_status kvarn_decode_attn(const kvarn_config *cfg, const kvarn_cache *cache,
                               const void *q, float *out, float softmax_scale,
                               void *workspace, size_t ws_bytes, void *stream);

/*
 * One decode step: kvarn_append_seal of (k_new, v_new) followed by
 * kvarn_decode_attn of q, with the same results and the same cache state
 * afterwards [P2 §2.1: a group is sealed when its last token arrives, before
 * anything attends over it; P2 §1: attention over the sealed groups and the
 * exact sink and tail].  k_new, v_new: device fp16 [batch][Hkv][D]; q, out,
 * softmax_scale, workspace, ws_bytes: as for kvarn_decode_attn.  len_host:
 * host int32 [batch] holding every request's seq_len before this step (the
 * caller's own count), or NULL.  When len_host shows that no request's token
 * completes a group and no request is at capacity, the append rides in the
 * decode launches (the split kernel reads the new token from k_new and
 * stores it in its sink or tail slot, the combine kernel advances seq_len):
 * two launches instead of three.  Otherwise (or with NULL) the step is the
 * three launches.  len_host must equal the cache's seq_len: with other
 * values the outputs are unspecified, and a request whose token would in
 * fact complete a group or find its cache full is left unchanged (its token
 * is not appended) rather than written to a wrong slot.  A negative value
 * returns KVARN_EINVAL before anything is queued.
 */
kvarn_status kvarn_decode_step(const kvarn_config *cfg, const kvarn_cache *cache,
                               const void *k_new, const void *v_new, const void *q, float *out,
                               float softmax_scale, const int32_t *len_host,
                               void *workspace, size_t ws_bytes, void *stream);

/*
 * kvarn_decode_attn without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, kernels and results as kvarn_decode_attn; the workspace is a
 * fixed device array of KVARN_NOALLOC_SCRATCH_BYTES inside the library, one
 * per device, held until the process ends.  A batch and capacity whose
 * workspace (kvarn_decode_workspace_bytes) exceeds it returns
 * KVARN_EWORKSPACE before anything is queued.  Every call on a device shares
 * that device's array: calls that overlap on one device (different streams,
 * or threads) race and must be serialized by the caller; calls in one stream
 * are ordered.  No state carries from one call to the next.
 */
#define KVARN_NOALLOC_SCRATCH_BYTES (16u << 20)
kvarn_status kvarn_decode_attn_noalloc(const kvarn_config *cfg, const kvarn_cache *cache,
                                       const void *q, float *out, float softmax_scale, void *stream);

/*
 * The two phases of kvarn_decode_attn, for callers that schedule them apart
 * (kvarn_decode_attn == partial then combine, same arguments):
 *   partial: the split-K kernel; writes per-split (max, sum, output) partials
 *            of every request and query head into `workspace`;
 *   combine: log-sum-exp merge of those partials, one inverse Hadamard of the
 *            record part per query head, normalization; writes `out`.
 * The workspace must not be touched between the two calls, and the cache
 * (seq_len included) must be unchanged.
 */
kvarn_status kvarn_decode_attn_partial(const kvarn_config *cfg, const kvarn_cache *cache, const void *q,
                                       float softmax_scale, void *workspace, size_t ws_bytes, void *stream);
kvarn_status kvarn_decode_attn_combine(const kvarn_config *cfg, const kvarn_cache *cache, float *out,
                                       void *workspace, size_t ws_bytes, void *stream);

/*
 * Chunked-prefill attention over the cache [P2 §2.1: attention paths read the
 * records directly; §7: the format's cost shows in prefill].  The chunk is
 * the last `chunk` cached positions of every request (append the chunk with
 * kvarn_prefill / kvarn_append first: every group it completed is sealed).
 * The query of position p = seq_len[b] - chunk + i (q: device fp16
 * [batch][chunk][Hq][D], post-RoPE) attends causally over positions 0..p as
 * the cache holds them: sink and tail exact, sealed groups through their
 * records, in the rotated frame with the output rotated back once [P2 §1].
 * Query head h reads KV head floor(h*Hkv/Hq).  out: device fp32
 * [batch][chunk][Hq][D]; rows whose position would be negative (chunk >
 * seq_len[b]) are left unwritten.  softmax_scale multiplies q.k.  No
 * workspace; chunk 0 queues nothing.
 */
kvarn_status kvarn_prefill_attn(const kvarn_config *cfg, const kvarn_cache *cache, const void *q,
                                int32_t chunk, float *out, float softmax_scale, void *stream);

/*
 * Seal n independent tiles (the same kernel as kvarn_seal_group).
 * src: device fp16 [n][128][D].  dst: device; tile i's record is written at
 * dst + i*dst_stride (dst_stride >= kvarn_record_bytes, multiple of 16).
 * kind 0 = K layout (token-major codes), 1 = V layout (channel-major).
 * dbg: NULL, or device fp32 [n][128 + D] receiving each tile's token scales
 * s_t and channel scales c_j before their fp16 rounding.
 */
kvarn_status kvarn_seal_tiles(int32_t head_dim, int32_t bits, int32_t kind, int32_t sinkhorn_iters,
                              const void *src, void *dst, int64_t dst_stride, float *dbg,
                              int32_t n, void *stream);

/*
 * Convert records to the standard fp16 layout [P2 §2.1: attention paths
 * that cannot read records convert them first].  For n records at
 * src + i*src_stride (kind 0 = K, 1 = V), writes the original-frame
 * reconstruction (s_t*(code-mid)*c_j, times H_D/sqrt(D)) rounded to fp16 into
 * dst (device fp16 [n][128][D]).
 */
kvarn_status kvarn_dequant_records(int32_t head_dim, int32_t bits, int32_t kind,
                                   const void *src, int64_t src_stride, void *dst,
                                   int32_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
