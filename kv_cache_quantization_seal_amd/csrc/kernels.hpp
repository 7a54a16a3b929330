// Internal launch interface between the C ABI (kvarn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

constexpr int kMaxPrefillBatch = 256;  // requests per prefill launch

// Code widths (bits); K and V take any two of them [every ordered pair is
// built: the seal kernels take the widths at run time, the decode split
// kernel has one instance per pair].
constexpr bool width_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }
constexpr bool pair_ok(int kb, int vb) { return width_ok(kb) && width_ok(vb); }
// Index of a width in 2, 3, 4, 5, 6, 8.
constexpr int width_index(int b) { return b == 8 ? 5 : b - 2; }

#define KVARN_DISPATCH_DB(D, B, CALL)                                                 \
  do {                                                                                \
    if (D == 128) {                                                                   \
      if (B == 2) CALL(128, 2); else if (B == 3) CALL(128, 3); else if (B == 4) CALL(128, 4); \
      else if (B == 5) CALL(128, 5); else if (B == 6) CALL(128, 6); else if (B == 8) CALL(128, 8); \
    } else {                                                                          \
      if (B == 2) CALL(256, 2); else if (B == 3) CALL(256, 3); else if (B == 4) CALL(256, 4); \
      else if (B == 5) CALL(256, 5); else if (B == 6) CALL(256, 6); else if (B == 8) CALL(256, 8); \
    }                                                                                 \
  } while (0)

// Where a cache's records live.  Contiguous (table NULL): the (K record,
// V record) pair of (request b, KV head h, group g) is pair number
// (b Hkv + h) max_groups + g of the records buffer.  Paged (the block table
// of a paged KV cache, one block per 128-token group holding the Hkv pairs of
// that group): pair number table[b max_groups + g] Hkv + h of a pool of
// num_blocks blocks.  A table entry outside [0, num_blocks) gives the group
// no storage: it is not written, and decoding treats it as absent.
struct RecordMap {
  const int32_t* table;
  int32_t num_blocks;
};

// Byte offset of the record pair of (b, h, g), or -1 if it has no storage.
// (b, g) are uniform over the calling workgroup: the table entry is a scalar
// load (its own counter, so waiting for it never waits for vector loads or
// stores in flight).
__device__ __forceinline__ int64_t pair_offset(const RecordMap& m, int b, int h, int g, int hkv, int max_groups,
                                               int64_t group_bytes) {
  if (!m.table) return (((int64_t)b * hkv + h) * max_groups + g) * group_bytes;
  typedef const __attribute__((address_space(4))) int32_t ConstTableEntry;
  const int blk = *(ConstTableEntry*)(m.table + (int64_t)b * max_groups + g);
  if (blk < 0 || blk >= m.num_blocks) return -1;
  return ((int64_t)blk * hkv + h) * group_bytes;
}

struct PrefillLens {
  int32_t len[kMaxPrefillBatch];
};

// One layer cache of a (multi-layer) prefill: its prompt K/V and its cache.
struct PrefillLayer {
  const __half* k;   // [B][Hkv][src_tokens][D]
  const __half* v;
  uint8_t* records;
  RecordMap map;
  __half* sink_k;
  __half* sink_v;
  __half* tail_k;
  __half* tail_v;
  int32_t* seq_len;
};
constexpr int kMaxPrefillLayers = 16;  // layers per launch (kernel-argument space)

struct SealPrefillArgs {
  int64_t src_tokens;
  int64_t group_bytes;
  int rec_k_bytes;
  int hkv;
  int max_groups;
  int b0;
  int iters;
  int k_bits;  // code widths of the K and V records
  int v_bits;
  int gmax;     // groups per (request, head) in this launch (set by the launcher)
  int nbh;      // requests * KV heads in this launch (set by the launcher)
  int n_tiles;  // 2 * n_layers * nbh * gmax (set by the launcher)
  int n_layers;
  PrefillLens lens;
  PrefillLayer layer[kMaxPrefillLayers];
};

struct SealStreamArgs {
  const __half* tail_k;
  const __half* tail_v;
  const int32_t* seq_len;
  const int32_t* req;    // NULL: workgroup x / hkv is the request (the predicate form)
  const int32_t* group;  // with req: the group each entry names
  int batch;
  uint8_t* records;
  RecordMap map;
  int64_t group_bytes;
  int rec_k_bytes;
  int hkv;
  int max_groups;
  int iters;
  int k_bits;  // code widths of the K and V records
  int v_bits;
};

// Append + seal in one launch.  While it runs, seq_len[b] carries a count of
// the request's workgroups that have read it in bits kArriveShift..30.
constexpr int kArriveShift = 23;
constexpr uint32_t kLenMask = (1u << kArriveShift) - 1;

struct AppendSealArgs {
  __half* sink_k;
  __half* sink_v;
  __half* tail_k;
  __half* tail_v;
  const __half* k_new;
  const __half* v_new;
  uint8_t* records;
  int32_t* seq_len;
  RecordMap map;
  int64_t group_bytes;
  int rec_k_bytes;
  int hkv;
  int max_groups;
  int cap;  // tokens a request can hold: 128 + 128 max_groups + 127
  int iters;
  int k_bits;  // code widths of the K and V records
  int v_bits;
};

struct CacheArgs {
  __half* sink_k;
  __half* sink_v;
  __half* tail_k;
  __half* tail_v;
  const uint8_t* records;
  RecordMap map;
  int32_t* seq_len;
  int batch;
  int hkv;
  int max_groups;
  int64_t group_bytes;
  int rec_k_bytes;
};

struct DecodeArgs {
  CacheArgs c;
  const __half* q;     // [B][Hq][D]
  float* out;          // [B][Hq][D]
  float* ws_o;         // [B][Hq][nsplit][D]
  float* ws_ml;        // [B][Hq][nsplit][2]
  float scale;         // softmax scale (applied to q.k)
  int hq;
  int nsplit;          // record splits + exact splits
  int n_rec_splits;
  int groups_per_split;
  int groups_per_wave;
  int record_first;    // grid order: record workgroups first (else exact ones)
  // Append folded into the step (both NULL: the cache already holds the
  // step's token): fp16 [B][Hkv][D], the token at position seq_len[b].  The
  // exact split that covers that position reads it from here and writes it
  // to its sink or tail slot; the combine kernel then sets seq_len[b] + 1.
  // Only for steps where no request completes a group or is at capacity.
  const __half* k_new;
  const __half* v_new;
};

struct PrefillAttnArgs {
  CacheArgs c;
  const __half* q;  // [B][chunk][Hq][D]
  float* out;       // [B][chunk][Hq][D]
  int chunk;        // queries per request: positions seq_len - chunk .. seq_len - 1
  int hq;
  float scale;      // softmax scale (applied to q.k)
  int k_bits;
  int v_bits;
};

struct DecodePlan {
  int groups_per_wave;
  int groups_per_split;
  int n_rec_splits;
  int n_exact_splits;
  int nsplit;
  int record_first;   // record workgroups first in the split kernel's grid
  size_t ws_bytes;
};

// Workgroups of the split kernel that can be resident at once is at most
// this (the workspace query, which has no device, plans with it).
constexpr int kMaxResidentWgs = 4096;

// cus: compute units of the launch's device, or 0 (a device-free plan, used
// for the workspace bound; rounding to whole workgroups per CU only ever
// removes splits).
DecodePlan plan_decode(int D, int kb, int hq, int hkv, int batch, int max_groups, int resident_wgs, int cus);
// Resident split workgroups on the current device for this configuration.
int decode_resident_wgs(int D, int kb, int vb, int gq);
// Compute units of the current device (0 if unknown).
int decode_cu_count();

hipError_t launch_seal_tiles(int D, int bits, int kind, const void* src, void* dst, int64_t stride, float* dbg, int n,
                             int iters, hipStream_t st);
hipError_t launch_seal_prefill(int D, const SealPrefillArgs& a, int max_groups_in_batch, int nbh, hipStream_t st);
// nbh = entries * hkv (entries = batch in the predicate form, n in the list form).
hipError_t launch_seal_stream(int D, const SealStreamArgs& a, int nbh, hipStream_t st);
hipError_t launch_append_seal(int D, const AppendSealArgs& a, int nbh, hipStream_t st);
hipError_t launch_append(int D, const CacheArgs& c, const void* k, const void* v, hipStream_t st);
// Sink and tail copies of a prompt into every layer of `a` (a.lens, a.b0,
// a.n_layers, a.layer[], a.hkv, a.src_tokens), nb requests.
hipError_t launch_prefill_copy(int D, const SealPrefillArgs& a, int nb, hipStream_t st);
// phases: 1 = split kernel (partials into the workspace), 2 = combine kernel, 3 = both.
hipError_t launch_decode(int D, int kb, int vb, int gq, const DecodeArgs& a, int phases, hipStream_t st);
// The split kernel for K width b (decode_k<b>.hip): launch, and the resident
// workgroups on device `dev`.
#define KVARN_DECLARE_SPLIT(b)                                                                  \
  hipError_t launch_split_k##b(int D, int vb, int gq, const DecodeArgs& a, hipStream_t st); \
  int resident_split_k##b(int D, int vb, int gq, int dev);
KVARN_DECLARE_SPLIT(2)
KVARN_DECLARE_SPLIT(3)
KVARN_DECLARE_SPLIT(4)
KVARN_DECLARE_SPLIT(5)
KVARN_DECLARE_SPLIT(6)
KVARN_DECLARE_SPLIT(8)
#undef KVARN_DECLARE_SPLIT
hipError_t launch_prefill_attn(int D, int gq, const PrefillAttnArgs& a, hipStream_t st);
hipError_t launch_dequant(int D, int bits, int kind, const void* src, int64_t src_stride, void* dst, int n,
                          hipStream_t st);

#ifdef KVARN_WAVE_TRACE
// Trace build only: copy (host non-NULL) or clear (host NULL) the per-wave
// timestamp buffer of the decode split kernel for K width b, of the seal
// kernels, or of the chunked-prefill attention kernel (see trace.hpp).
hipError_t trace_io_decode_k2(void* host, size_t bytes);
hipError_t trace_io_decode_k3(void* host, size_t bytes);
hipError_t trace_io_decode_k4(void* host, size_t bytes);
hipError_t trace_io_decode_k5(void* host, size_t bytes);
hipError_t trace_io_decode_k6(void* host, size_t bytes);
hipError_t trace_io_decode_k8(void* host, size_t bytes);
hipError_t trace_io_seal(void* host, size_t bytes);
hipError_t trace_io_prefill_attn(void* host, size_t bytes);
#endif

}  // namespace kvarn
