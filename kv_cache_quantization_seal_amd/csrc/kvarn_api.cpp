// C ABI of the KVarN hot path: host-side validation and kernel dispatch.
// Every argument check runs before anything is queued, so a rejected call
// leaves the GPU untouched (and needs no GPU at all).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/kvarn.h"
#include "kernels.hpp"

// Scratch of kvarn_decode_attn_noalloc: the decode workspace (per-split
// partial outputs, maxima and sums) in a file-scope device array, so that
// entry point needs no allocation.  Each device holds its own copy for the
// life of the process; host code reaches it only through the address
// hipGetSymbolAddress returns on that device.
constexpr size_t kNoAllocScratchBytes = (size_t)KVARN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512] = "";

kvarn_status fail(kvarn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kvarn_status ok() {
  g_err[0] = '\0';
  return KVARN_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool bits_ok(int b) { return kvarn::width_ok(b); }
bool dim_ok(int d) { return d == 128 || d == 256; }

kvarn_status check_cfg(const kvarn_config* c) {
  if (!c) return fail(KVARN_EINVAL, "config is NULL");
  if (c->group != KVARN_GROUP || c->sink != KVARN_SINK)
    return fail(KVARN_EUNSUPPORTED, "group and sink must both be 128 (got %d, %d)", c->group, c->sink);
  if (!dim_ok(c->head_dim)) return fail(KVARN_EUNSUPPORTED, "head_dim must be 128 or 256 (got %d)", c->head_dim);
  if (!bits_ok(c->k_bits) || !bits_ok(c->v_bits))
    return fail(KVARN_EUNSUPPORTED, "k_bits and v_bits must be 2, 3, 4, 5, 6 or 8 (got %d, %d)", c->k_bits,
                c->v_bits);
  if (c->num_q_heads <= 0 || c->num_kv_heads <= 0)
    return fail(KVARN_EINVAL, "head counts must be positive (got %d, %d)", c->num_q_heads, c->num_kv_heads);
  if (c->num_q_heads % c->num_kv_heads)
    return fail(KVARN_EINVAL, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", c->num_q_heads,
                c->num_kv_heads);
  const int g = c->num_q_heads / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4)
    return fail(KVARN_EUNSUPPORTED, "query heads per KV head must be 1, 2 or 4 (got %d)", g);
  if (c->sinkhorn_iters < 0 || c->sinkhorn_iters > 64)
    return fail(KVARN_EINVAL, "sinkhorn_iters must be in [0, 64] (got %d)", c->sinkhorn_iters);
  return KVARN_OK;
}

size_t rec_bytes(int d, int bits) { return (size_t)KVARN_GROUP * d * bits / 8 + 2 * KVARN_GROUP + 2 * (size_t)d; }

kvarn_status check_cache(const kvarn_config* c, const kvarn_cache* k) {
  if (!k) return fail(KVARN_EINVAL, "cache is NULL");
  if (k->batch <= 0) return fail(KVARN_EINVAL, "cache batch must be positive (got %d)", k->batch);
  if (k->max_groups < 0) return fail(KVARN_EINVAL, "cache max_groups must be >= 0 (got %d)", k->max_groups);
  if (!k->sink_k || !k->sink_v || !k->tail_k || !k->tail_v || !k->seq_len)
    return fail(KVARN_EINVAL, "cache sink/tail/seq_len pointers must be non-NULL");
  if (k->max_groups > 0 && !k->records) return fail(KVARN_EINVAL, "cache records is NULL");
  if (k->block_table) {
    if (k->num_blocks <= 0)
      return fail(KVARN_EINVAL, "a paged cache needs num_blocks > 0 (got %d)", k->num_blocks);
    if (!aligned(k->block_table, 4)) return fail(KVARN_EINVAL, "cache block_table must be 4-byte aligned");
  }
  if (!aligned(k->sink_k, 16) || !aligned(k->sink_v, 16) || !aligned(k->tail_k, 16) || !aligned(k->tail_v, 16) ||
      !aligned(k->records, 16) || !aligned(k->seq_len, 4))
    return fail(KVARN_EINVAL, "cache buffers must be 16-byte aligned");
  (void)c;
  return KVARN_OK;
}

kvarn::RecordMap record_map(const kvarn_cache* k) {
  kvarn::RecordMap m;
  m.table = k->block_table;
  m.num_blocks = k->block_table ? k->num_blocks : 0;
  return m;
}

kvarn::CacheArgs cache_args(const kvarn_config* c, const kvarn_cache* k) {
  kvarn::CacheArgs a;
  a.sink_k = (__half*)k->sink_k;
  a.sink_v = (__half*)k->sink_v;
  a.tail_k = (__half*)k->tail_k;
  a.tail_v = (__half*)k->tail_v;
  a.records = (const uint8_t*)k->records;
  a.map = record_map(k);
  a.seq_len = k->seq_len;
  a.batch = k->batch;
  a.hkv = c->num_kv_heads;
  a.max_groups = k->max_groups;
  a.rec_k_bytes = (int)rec_bytes(c->head_dim, c->k_bits);
  a.group_bytes = (int64_t)a.rec_k_bytes + (int64_t)rec_bytes(c->head_dim, c->v_bits);
  return a;
}

kvarn_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVARN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

kvarn_status kvarn_check_config(const kvarn_config* cfg) {
  const kvarn_status s = check_cfg(cfg);
  return s == KVARN_OK ? ok() : s;
}

size_t kvarn_record_bytes(int32_t head_dim, int32_t bits) {
  if (!dim_ok(head_dim) || !bits_ok(bits)) return 0;
  return rec_bytes(head_dim, bits);
}

size_t kvarn_group_bytes(const kvarn_config* cfg) {
  if (check_cfg(cfg) != KVARN_OK) return 0;
  return rec_bytes(cfg->head_dim, cfg->k_bits) + rec_bytes(cfg->head_dim, cfg->v_bits);
}

size_t kvarn_decode_workspace_bytes(const kvarn_config* cfg, int32_t batch, int32_t max_groups) {
  if (check_cfg(cfg) != KVARN_OK || batch <= 0 || max_groups < 0) return 0;
  // Planned for the most resident workgroups any device allows: a launch
  // plans for fewer, hence fewer splits and no more workspace.
  return kvarn::plan_decode(cfg->head_dim, cfg->k_bits, cfg->num_q_heads, cfg->num_kv_heads, batch, max_groups,
                            kvarn::kMaxResidentWgs, 0)
      .ws_bytes;
}

kvarn_status kvarn_decode_plan(const kvarn_config* cfg, int32_t batch, int32_t max_groups, int32_t* out) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if (!out) return fail(KVARN_EINVAL, "out must be non-NULL");
  if (batch <= 0 || max_groups < 0) return fail(KVARN_EINVAL, "batch must be > 0 and max_groups >= 0");
  const int resident = kvarn::decode_resident_wgs(cfg->head_dim, cfg->k_bits, cfg->v_bits,
                                                  cfg->num_q_heads / cfg->num_kv_heads);
  const kvarn::DecodePlan p = kvarn::plan_decode(cfg->head_dim, cfg->k_bits, cfg->num_q_heads, cfg->num_kv_heads, batch,
                                                 max_groups, resident, kvarn::decode_cu_count());
  const int64_t pairs = (int64_t)batch * cfg->num_kv_heads;
  out[0] = p.n_rec_splits;
  out[1] = p.n_exact_splits;
  out[2] = p.groups_per_wave;
  out[3] = (int32_t)(pairs * p.n_rec_splits);
  out[4] = (int32_t)(pairs * p.n_exact_splits);
  return ok();
}

const char* kvarn_last_error(void) { return g_err; }

const char* kvarn_status_string(kvarn_status s) {
  switch (s) {
    case KVARN_OK: return "KVARN_OK";
    case KVARN_EINVAL: return "KVARN_EINVAL";
    case KVARN_EUNSUPPORTED: return "KVARN_EUNSUPPORTED";
    case KVARN_ERANGE: return "KVARN_ERANGE";
    case KVARN_EWORKSPACE: return "KVARN_EWORKSPACE";
    case KVARN_EHIP: return "KVARN_EHIP";
  }
  return "KVARN_UNKNOWN";
}

kvarn_status kvarn_append(const kvarn_config* cfg, const kvarn_cache* cache, const void* k_new, const void* v_new,
                          void* stream) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVARN_OK) return s;
  if (!k_new || !v_new) return fail(KVARN_EINVAL, "k_new and v_new must be non-NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(KVARN_EINVAL, "k_new and v_new must be 16-byte aligned");
  return hip_status(kvarn::launch_append(cfg->head_dim, cache_args(cfg, cache), k_new, v_new, (hipStream_t)stream),
                    "kvarn_append launch");
}

kvarn_status kvarn_append_seal(const kvarn_config* cfg, const kvarn_cache* cache, const void* k_new,
                               const void* v_new, void* stream) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVARN_OK) return s;
  if (!k_new || !v_new) return fail(KVARN_EINVAL, "k_new and v_new must be non-NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(KVARN_EINVAL, "k_new and v_new must be 16-byte aligned");
  const int64_t cap = (int64_t)KVARN_SINK + (int64_t)KVARN_GROUP * cache->max_groups + KVARN_GROUP - 1;
  if (cap > (int64_t)kvarn::kLenMask)
    return fail(KVARN_ERANGE, "kvarn_append_seal needs a capacity below 2^%d tokens (max_groups %d is too large)",
                kvarn::kArriveShift, cache->max_groups);
  if (2 * cfg->num_kv_heads >= (1 << (31 - kvarn::kArriveShift)))
    return fail(KVARN_EUNSUPPORTED, "kvarn_append_seal supports at most %d KV heads",
                (1 << (31 - kvarn::kArriveShift)) / 2 - 1);
  const int64_t nbh = (int64_t)cache->batch * cfg->num_kv_heads;
  if (nbh > 0x7fffffff) return fail(KVARN_ERANGE, "batch * num_kv_heads too large");
  const kvarn::CacheArgs c = cache_args(cfg, cache);
  kvarn::AppendSealArgs a;
  a.sink_k = c.sink_k;
  a.sink_v = c.sink_v;
  a.tail_k = c.tail_k;
  a.tail_v = c.tail_v;
  a.k_new = (const __half*)k_new;
  a.v_new = (const __half*)v_new;
  a.records = (uint8_t*)cache->records;
  a.map = c.map;
  a.seq_len = cache->seq_len;
  a.group_bytes = c.group_bytes;
  a.rec_k_bytes = c.rec_k_bytes;
  a.hkv = c.hkv;
  a.max_groups = c.max_groups;
  a.cap = (int)cap;
  a.iters = cfg->sinkhorn_iters;
  a.k_bits = cfg->k_bits;
  a.v_bits = cfg->v_bits;
  return hip_status(kvarn::launch_append_seal(cfg->head_dim, a, (int)nbh, (hipStream_t)stream),
                    "kvarn_append_seal launch");
}

kvarn_status kvarn_seal_group(const kvarn_config* cfg, const kvarn_cache* cache, const int32_t* d_req,
                              const int32_t* d_group, int32_t n, void* stream) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVARN_OK) return s;
  if (n < 0) return fail(KVARN_EINVAL, "n must be >= 0 (got %d)", n);
  if (n == 0) return ok();  // an empty list (its pointers may be NULL): nothing to queue
  if (!d_req != !d_group) return fail(KVARN_EINVAL, "d_req and d_group must both be NULL or both be non-NULL");
  if (!d_req && n != cache->batch)
    return fail(KVARN_EINVAL, "the predicate form (d_req NULL) needs n == batch (got n %d, batch %d)", n,
                cache->batch);
  if (d_req && (!aligned(d_req, 4) || !aligned(d_group, 4)))
    return fail(KVARN_EINVAL, "d_req and d_group must be 4-byte aligned");
  if (cache->max_groups == 0) return ok();
  const int64_t nbh = (int64_t)n * cfg->num_kv_heads;
  if (nbh > 0x7fffffff) return fail(KVARN_ERANGE, "n * num_kv_heads too large");
  const kvarn::CacheArgs c = cache_args(cfg, cache);
  kvarn::SealStreamArgs a;
  a.tail_k = c.tail_k;
  a.tail_v = c.tail_v;
  a.seq_len = c.seq_len;
  a.req = d_req;
  a.group = d_group;
  a.batch = cache->batch;
  a.records = (uint8_t*)cache->records;
  a.map = c.map;
  a.group_bytes = c.group_bytes;
  a.rec_k_bytes = c.rec_k_bytes;
  a.hkv = c.hkv;
  a.max_groups = c.max_groups;
  a.iters = cfg->sinkhorn_iters;
  a.k_bits = cfg->k_bits;
  a.v_bits = cfg->v_bits;
  return hip_status(kvarn::launch_seal_stream(cfg->head_dim, a, (int)nbh, (hipStream_t)stream),
                    "kvarn_seal_group launch");
}

kvarn_status kvarn_prefill_layers(const kvarn_config* cfg, const kvarn_cache* caches, int32_t n_layers,
                                  const void* const* k, const void* const* v, int64_t src_tokens,
                                  const int32_t* len_host, void* stream) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if (n_layers < 0) return fail(KVARN_EINVAL, "n_layers must be >= 0 (got %d)", n_layers);
  if (n_layers == 0) return ok();
  if (!caches || !k || !v || !len_host) return fail(KVARN_EINVAL, "caches, k, v and len_host must be non-NULL");
  for (int l = 0; l < n_layers; ++l) {
    if ((s = check_cache(cfg, &caches[l])) != KVARN_OK) return s;
    if (caches[l].batch != caches[0].batch || caches[l].max_groups != caches[0].max_groups)
      return fail(KVARN_EINVAL, "layer %d: every layer cache must have the batch and max_groups of layer 0", l);
    if (!k[l] || !v[l]) return fail(KVARN_EINVAL, "layer %d: k and v must be non-NULL", l);
    if (!aligned(k[l], 16) || !aligned(v[l], 16))
      return fail(KVARN_EINVAL, "layer %d: k and v must be 16-byte aligned", l);
  }
  if (src_tokens < 0) return fail(KVARN_EINVAL, "src_tokens must be >= 0");
  const kvarn_cache* c0 = &caches[0];
  const int64_t cap = (int64_t)KVARN_SINK + (int64_t)KVARN_GROUP * c0->max_groups + KVARN_GROUP - 1;
  for (int b = 0; b < c0->batch; ++b) {
    if (len_host[b] < 0) return fail(KVARN_EINVAL, "len_host[%d] = %d is negative", b, len_host[b]);
    if (len_host[b] > src_tokens)
      return fail(KVARN_ERANGE, "len_host[%d] = %d exceeds src_tokens = %lld", b, len_host[b], (long long)src_tokens);
    if (len_host[b] > cap)
      return fail(KVARN_ERANGE, "len_host[%d] = %d exceeds the cache capacity %lld", b, len_host[b], (long long)cap);
  }
  const kvarn::CacheArgs c = cache_args(cfg, c0);
  hipStream_t st = (hipStream_t)stream;
  for (int l0 = 0; l0 < n_layers; l0 += kvarn::kMaxPrefillLayers) {
    const int nl = n_layers - l0 < kvarn::kMaxPrefillLayers ? n_layers - l0 : kvarn::kMaxPrefillLayers;
    kvarn::SealPrefillArgs a;
    memset(&a, 0, sizeof(a));
    a.src_tokens = src_tokens;
    a.group_bytes = c.group_bytes;
    a.rec_k_bytes = c.rec_k_bytes;
    a.hkv = c.hkv;
    a.max_groups = c.max_groups;
    a.iters = cfg->sinkhorn_iters;
    a.k_bits = cfg->k_bits;
    a.v_bits = cfg->v_bits;
    a.n_layers = nl;
    for (int i = 0; i < nl; ++i) {
      const kvarn_cache* ci = &caches[l0 + i];
      kvarn::PrefillLayer& L = a.layer[i];
      L.k = (const __half*)k[l0 + i];
      L.v = (const __half*)v[l0 + i];
      L.records = (uint8_t*)ci->records;
      L.map = record_map(ci);
      L.sink_k = (__half*)ci->sink_k;
      L.sink_v = (__half*)ci->sink_v;
      L.tail_k = (__half*)ci->tail_k;
      L.tail_v = (__half*)ci->tail_v;
      L.seq_len = ci->seq_len;
    }
    for (int b0 = 0; b0 < c0->batch; b0 += kvarn::kMaxPrefillBatch) {
      const int nb = c0->batch - b0 < kvarn::kMaxPrefillBatch ? c0->batch - b0 : kvarn::kMaxPrefillBatch;
      memset(&a.lens, 0, sizeof(a.lens));
      int max_g = 0;
      for (int i = 0; i < nb; ++i) {
        a.lens.len[i] = len_host[b0 + i];
        const int g = a.lens.len[i] > KVARN_SINK ? (a.lens.len[i] - KVARN_SINK) / KVARN_GROUP : 0;
        if (g > max_g) max_g = g;
      }
      a.b0 = b0;
      hipError_t e = kvarn::launch_prefill_copy(cfg->head_dim, a, nb, st);
      if (e != hipSuccess) return hip_status(e, "kvarn_prefill copy launch");
      if (max_g > 0) {
        // The seal launch walks 2 * layers * nb * Hkv * max_g tiles with int indices.
        if ((int64_t)2 * nl * nb * c.hkv * max_g >= ((int64_t)1 << 30))
          return fail(KVARN_ERANGE, "prefill of %d layers x %d requests x %d KV heads x %d groups is too large", nl,
                      nb, c.hkv, max_g);
        e = kvarn::launch_seal_prefill(cfg->head_dim, a, max_g, nb * c.hkv, st);
        if (e != hipSuccess) return hip_status(e, "kvarn_prefill seal launch");
      }
    }
  }
  return ok();
}

kvarn_status kvarn_prefill(const kvarn_config* cfg, const kvarn_cache* cache, const void* k, const void* v,
                           int64_t src_tokens, const int32_t* len_host, void* stream) {
  if (!cache) return fail(KVARN_EINVAL, "cache is NULL");
  if (!k || !v) return fail(KVARN_EINVAL, "k, v and len_host must be non-NULL");
  return kvarn_prefill_layers(cfg, cache, 1, &k, &v, src_tokens, len_host, stream);
}

static kvarn_status decode_common(const kvarn_config* cfg, const kvarn_cache* cache, const void* q, float* out,
                                  float softmax_scale, void* workspace, size_t ws_bytes, int phases, void* stream,
                                  const char* what, const void* k_new = nullptr, const void* v_new = nullptr) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVARN_OK) return s;
  if ((phases & 1) && !q) return fail(KVARN_EINVAL, "q must be non-NULL");
  if ((phases & 2) && !out) return fail(KVARN_EINVAL, "out must be non-NULL");
  if ((q && !aligned(q, 16)) || (out && !aligned(out, 16)))
    return fail(KVARN_EINVAL, "q and out must be 16-byte aligned");
  const int resident = kvarn::decode_resident_wgs(cfg->head_dim, cfg->k_bits, cfg->v_bits,
                                                  cfg->num_q_heads / cfg->num_kv_heads);
  const kvarn::DecodePlan p = kvarn::plan_decode(cfg->head_dim, cfg->k_bits, cfg->num_q_heads, cfg->num_kv_heads, cache->batch,
                                                 cache->max_groups, resident, kvarn::decode_cu_count());
  if (!workspace || ws_bytes < p.ws_bytes)
    return fail(KVARN_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, p.ws_bytes);
  if (!aligned(workspace, 256)) return fail(KVARN_EINVAL, "workspace must be 256-byte aligned");
  if (!(softmax_scale == softmax_scale)) return fail(KVARN_EINVAL, "softmax_scale is NaN");
  kvarn::DecodeArgs a;
  a.c = cache_args(cfg, cache);
  a.q = (const __half*)q;
  a.out = out;
  const size_t rows = (size_t)cache->batch * cfg->num_q_heads * p.nsplit;
  const size_t o_bytes = (rows * cfg->head_dim * sizeof(float) + 255) & ~(size_t)255;
  a.ws_o = (float*)workspace;
  a.ws_ml = (float*)((char*)workspace + o_bytes);
  a.scale = softmax_scale;
  a.hq = cfg->num_q_heads;
  a.nsplit = p.nsplit;
  a.n_rec_splits = p.n_rec_splits;
  a.groups_per_split = p.groups_per_split;
  a.groups_per_wave = p.groups_per_wave;
  a.record_first = p.record_first;
  a.k_new = (const __half*)k_new;
  a.v_new = (const __half*)v_new;
  return hip_status(kvarn::launch_decode(cfg->head_dim, cfg->k_bits, cfg->v_bits,
                                         cfg->num_q_heads / cfg->num_kv_heads, a, phases, (hipStream_t)stream),
                    what);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
static void* scratch_ptr(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (!p) {
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptrs[dev].store(p, std::memory_order_release);
  }
  return p;
}

kvarn_status kvarn_decode_attn_noalloc(const kvarn_config* cfg, const kvarn_cache* cache, const void* q, float* out,
                                       float softmax_scale, void* stream) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVARN_OK) return s;
  if (!q || !out) return fail(KVARN_EINVAL, "q and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(KVARN_EINVAL, "q and out must be 16-byte aligned");
  if (!(softmax_scale == softmax_scale)) return fail(KVARN_EINVAL, "softmax_scale is NaN");
  const int resident = kvarn::decode_resident_wgs(cfg->head_dim, cfg->k_bits, cfg->v_bits,
                                                  cfg->num_q_heads / cfg->num_kv_heads);
  const kvarn::DecodePlan p = kvarn::plan_decode(cfg->head_dim, cfg->k_bits, cfg->num_q_heads, cfg->num_kv_heads, cache->batch,
                                                 cache->max_groups, resident, kvarn::decode_cu_count());
  if (p.ws_bytes > kNoAllocScratchBytes)
    return fail(KVARN_EWORKSPACE,
                "kvarn_decode_attn_noalloc: this batch and capacity need %zu bytes of decode scratch, more than "
                "the library's fixed %zu bytes (use kvarn_decode_attn with a workspace)",
                p.ws_bytes, kNoAllocScratchBytes);
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws) return fail(KVARN_EHIP, "kvarn_decode_attn_noalloc: scratch lookup: %s", hipGetErrorString(e));
  return decode_common(cfg, cache, q, out, softmax_scale, ws, kNoAllocScratchBytes, 3, stream,
                       "kvarn_decode_attn_noalloc launch");
}

kvarn_status kvarn_decode_attn(const kvarn_config* cfg, const kvarn_cache* cache, const void* q, float* out,
                               float softmax_scale, void* workspace, size_t ws_bytes, void* stream) {
  return decode_common(cfg, cache, q, out, softmax_scale, workspace, ws_bytes, 3, stream, "kvarn_decode_attn launch");
}

kvarn_status kvarn_decode_step(const kvarn_config* cfg, const kvarn_cache* cache, const void* k_new,
                               const void* v_new, const void* q, float* out, float softmax_scale,
                               const int32_t* len_host, void* workspace, size_t ws_bytes, void* stream) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVARN_OK) return s;
  if (!k_new || !v_new) return fail(KVARN_EINVAL, "k_new and v_new must be non-NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(KVARN_EINVAL, "k_new and v_new must be 16-byte aligned");
  // The append rides in the decode launches only if no request's token
  // completes a group (that group's seal must come before the attention)
  // and no request is at capacity (its append is skipped).
  bool fold = len_host != nullptr;
  if (fold) {
    const int64_t cap = (int64_t)KVARN_SINK + (int64_t)KVARN_GROUP * cache->max_groups + KVARN_GROUP - 1;
    for (int32_t b = 0; b < cache->batch; ++b) {
      const int64_t n = len_host[b];
      if (n < 0) return fail(KVARN_EINVAL, "len_host[%d] = %lld is negative", b, (long long)n);
      const int64_t n1 = n + 1;
      if (n >= cap || (n1 >= KVARN_SINK + KVARN_GROUP && (n1 - KVARN_SINK) % KVARN_GROUP == 0)) fold = false;
    }
  }
  if (!fold) {
    if ((s = kvarn_append_seal(cfg, cache, k_new, v_new, stream)) != KVARN_OK) return s;
    return decode_common(cfg, cache, q, out, softmax_scale, workspace, ws_bytes, 3, stream,
                         "kvarn_decode_step launch");
  }
  return decode_common(cfg, cache, q, out, softmax_scale, workspace, ws_bytes, 3, stream,
                       "kvarn_decode_step launch", k_new, v_new);
}

kvarn_status kvarn_decode_attn_partial(const kvarn_config* cfg, const kvarn_cache* cache, const void* q,
                                       float softmax_scale, void* workspace, size_t ws_bytes, void* stream) {
  return decode_common(cfg, cache, q, nullptr, softmax_scale, workspace, ws_bytes, 1, stream,
                       "kvarn_decode_attn_partial launch");
}

kvarn_status kvarn_decode_attn_combine(const kvarn_config* cfg, const kvarn_cache* cache, float* out, void* workspace,
                                       size_t ws_bytes, void* stream) {
  return decode_common(cfg, cache, nullptr, out, 1.0f, workspace, ws_bytes, 2, stream,
                       "kvarn_decode_attn_combine launch");
}

kvarn_status kvarn_prefill_attn(const kvarn_config* cfg, const kvarn_cache* cache, const void* q, int32_t chunk,
                                float* out, float softmax_scale, void* stream) {
  kvarn_status s = check_cfg(cfg);
  if (s != KVARN_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVARN_OK) return s;
  if (chunk < 0) return fail(KVARN_EINVAL, "chunk must be >= 0 (got %d)", chunk);
  if (chunk == 0) return ok();
  if (!q || !out) return fail(KVARN_EINVAL, "q and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(KVARN_EINVAL, "q and out must be 16-byte aligned");
  if (!(softmax_scale == softmax_scale)) return fail(KVARN_EINVAL, "softmax_scale is NaN");
  const int64_t cap = (int64_t)KVARN_SINK + (int64_t)KVARN_GROUP * cache->max_groups + KVARN_GROUP - 1;
  if (chunk > cap) return fail(KVARN_ERANGE, "chunk %d exceeds the cache capacity %lld", chunk, (long long)cap);
  const int gq = cfg->num_q_heads / cfg->num_kv_heads;
  if ((int64_t)cache->batch * cfg->num_kv_heads > 65535 || cache->batch > 65535)
    return fail(KVARN_ERANGE, "batch and KV heads exceed the launch grid");
  kvarn::PrefillAttnArgs a;
  a.c = cache_args(cfg, cache);
  a.q = (const __half*)q;
  a.out = out;
  a.chunk = chunk;
  a.hq = cfg->num_q_heads;
  a.scale = softmax_scale;
  a.k_bits = cfg->k_bits;
  a.v_bits = cfg->v_bits;
  return hip_status(kvarn::launch_prefill_attn(cfg->head_dim, gq, a, (hipStream_t)stream),
                    "kvarn_prefill_attn launch");
}

kvarn_status kvarn_seal_tiles(int32_t head_dim, int32_t bits, int32_t kind, int32_t sinkhorn_iters, const void* src,
                              void* dst, int64_t dst_stride, float* dbg, int32_t n, void* stream) {
  if (!dim_ok(head_dim)) return fail(KVARN_EUNSUPPORTED, "head_dim must be 128 or 256 (got %d)", head_dim);
  if (!bits_ok(bits)) return fail(KVARN_EUNSUPPORTED, "bits must be 2, 3, 4, 5, 6 or 8 (got %d)", bits);
  if (kind != 0 && kind != 1) return fail(KVARN_EINVAL, "kind must be 0 (K) or 1 (V) (got %d)", kind);
  if (sinkhorn_iters < 0 || sinkhorn_iters > 64) return fail(KVARN_EINVAL, "sinkhorn_iters must be in [0, 64]");
  if (n < 0) return fail(KVARN_EINVAL, "n must be >= 0");
  if (n == 0) return ok();
  if (!src || !dst) return fail(KVARN_EINVAL, "src and dst must be non-NULL");
  if (!aligned(src, 16) || !aligned(dst, 16) || (dbg && !aligned(dbg, 4)))
    return fail(KVARN_EINVAL, "src and dst must be 16-byte aligned");
  if (dst_stride < (int64_t)rec_bytes(head_dim, bits) || dst_stride % 16)
    return fail(KVARN_EINVAL, "dst_stride must be >= the record size and a multiple of 16");
  return hip_status(kvarn::launch_seal_tiles(head_dim, bits, kind, src, dst, dst_stride, dbg, n, sinkhorn_iters,
                                             (hipStream_t)stream),
                    "kvarn_seal_tiles launch");
}

kvarn_status kvarn_dequant_records(int32_t head_dim, int32_t bits, int32_t kind, const void* src, int64_t src_stride,
                                   void* dst, int32_t n, void* stream) {
  if (!dim_ok(head_dim)) return fail(KVARN_EUNSUPPORTED, "head_dim must be 128 or 256 (got %d)", head_dim);
  if (!bits_ok(bits)) return fail(KVARN_EUNSUPPORTED, "bits must be 2, 3, 4, 5, 6 or 8 (got %d)", bits);
  if (kind != 0 && kind != 1) return fail(KVARN_EINVAL, "kind must be 0 (K) or 1 (V) (got %d)", kind);
  if (n < 0) return fail(KVARN_EINVAL, "n must be >= 0");
  if (n == 0) return ok();
  if (!src || !dst) return fail(KVARN_EINVAL, "src and dst must be non-NULL");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(KVARN_EINVAL, "src and dst must be 16-byte aligned");
  if (src_stride < (int64_t)rec_bytes(head_dim, bits) || src_stride % 16)
    return fail(KVARN_EINVAL, "src_stride must be >= the record size and a multiple of 16");
  return hip_status(kvarn::launch_dequant(head_dim, bits, kind, src, src_stride, dst, n, (hipStream_t)stream),
                    "kvarn_dequant_records launch");
}

#ifdef KVARN_WAVE_TRACE
// Trace build (libkvarn_trace.so) only, not part of the KVarN ABI: per-wave
// phase timestamps of the bulk seal kernel (which 1) or of the decode split
// kernel for K width b (which 100 + b).  host NULL clears the buffer;
// otherwise copies `bytes` bytes of it.  Synchronous; returns 0 or a HIP
// error code (hipErrorInvalidValue for an unknown `which`).
int kvarn_trace_io(int which, void* host, size_t bytes) {
  switch (which) {
    case 1: return (int)kvarn::trace_io_seal(host, bytes);
    case 2: return (int)kvarn::trace_io_prefill_attn(host, bytes);
    case 102: return (int)kvarn::trace_io_decode_k2(host, bytes);
    case 103: return (int)kvarn::trace_io_decode_k3(host, bytes);
    case 104: return (int)kvarn::trace_io_decode_k4(host, bytes);
    case 105: return (int)kvarn::trace_io_decode_k5(host, bytes);
    case 106: return (int)kvarn::trace_io_decode_k6(host, bytes);
    case 108: return (int)kvarn::trace_io_decode_k8(host, bytes);
  }
  return (int)hipErrorInvalidValue;
}
#endif

}  // extern "C"
