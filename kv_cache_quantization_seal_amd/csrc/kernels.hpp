// Internal launch interface between the C ABI (kvarn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

constexpr int kMaxPrefillBatch = 256;  // requests per prefill launch

// Code widths (bits) and the (K, V) width pairs the kernels are built for:
// every symmetric width, the pairs of widths 2 and 4, and the asymmetric
// presets 3-2, 5-4 and 6-5.
constexpr bool width_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }
constexpr bool pair_ok(int kb, int vb) {
  return (kb == vb && width_ok(kb)) || (kb == 2 && vb == 4) || (kb == 4 && vb == 2) || (kb == 3 && vb == 2) ||
         (kb == 5 && vb == 4) || (kb == 6 && vb == 5);
}
// Index of a width in 2, 3, 4, 5, 6, 8.
constexpr int width_index(int b) { return b == 8 ? 5 : b - 2; }

// CALL(d, kb, vb) for the instance matching (D, KB, VB); nothing for a pair
// that pair_ok rejects (the host checks first).
#define KVARN_PAIRS_FOR_D(d, KB, VB, CALL)      \
  if (KB == 2 && VB == 2) CALL(d, 2, 2);        \
  else if (KB == 2 && VB == 4) CALL(d, 2, 4);   \
  else if (KB == 4 && VB == 2) CALL(d, 4, 2);   \
  else if (KB == 4 && VB == 4) CALL(d, 4, 4);   \
  else if (KB == 3 && VB == 3) CALL(d, 3, 3);   \
  else if (KB == 5 && VB == 5) CALL(d, 5, 5);   \
  else if (KB == 6 && VB == 6) CALL(d, 6, 6);   \
  else if (KB == 8 && VB == 8) CALL(d, 8, 8);   \
  else if (KB == 3 && VB == 2) CALL(d, 3, 2);   \
  else if (KB == 5 && VB == 4) CALL(d, 5, 4);   \
  else if (KB == 6 && VB == 5) CALL(d, 6, 5);
#define KVARN_DISPATCH_DKV(D, KB, VB, CALL)     \
  do {                                          \
    if (D == 128) {                             \
      KVARN_PAIRS_FOR_D(128, KB, VB, CALL)      \
    } else {                                    \
      KVARN_PAIRS_FOR_D(256, KB, VB, CALL)      \
    }                                           \
  } while (0)
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
__device__ __forceinline__ int64_t pair_offset(const RecordMap& m, int b, int h, int g, int hkv, int max_groups,
                                               int64_t group_bytes) {
  if (!m.table) return (((int64_t)b * hkv + h) * max_groups + g) * group_bytes;
  const int blk = m.table[(int64_t)b * max_groups + g];
  if (blk < 0 || blk >= m.num_blocks) return -1;
  return ((int64_t)blk * hkv + h) * group_bytes;
}

struct PrefillLens {
  int32_t len[kMaxPrefillBatch];
};

struct SealPrefillArgs {
  const __half* k;
  const __half* v;
  int64_t src_tokens;
  uint8_t* records;
  RecordMap map;
  int64_t group_bytes;
  int rec_k_bytes;
  int hkv;
  int max_groups;
  int b0;
  int iters;
  int gmax;     // groups per (request, head) in this launch (set by the launcher)
  int nbh;      // requests * KV heads in this launch (set by the launcher)
  int n_tiles;  // 2 * nbh * gmax (set by the launcher)
  PrefillLens lens;
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
};

struct DecodePlan {
  int groups_per_wave;
  int groups_per_split;
  int n_rec_splits;
  int n_exact_splits;
  int nsplit;
  size_t ws_bytes;
};

// Workgroups of the split kernel that can be resident at once is at most
// this (the workspace query, which has no device, plans with it).
constexpr int kMaxResidentWgs = 4096;

// cus: compute units of the launch's device, or 0 (a device-free plan, used
// for the workspace bound; rounding to whole workgroups per CU only ever
// removes splits).
DecodePlan plan_decode(int D, int hq, int hkv, int batch, int max_groups, int resident_wgs, int cus);
// Resident split workgroups on the current device for this configuration.
int decode_resident_wgs(int D, int kb, int vb, int gq);
// Compute units of the current device (0 if unknown).
int decode_cu_count();

hipError_t launch_seal_tiles(int D, int bits, int kind, const void* src, void* dst, int64_t stride, float* dbg, int n,
                             int iters, hipStream_t st);
hipError_t launch_seal_prefill(int D, int kb, int vb, const SealPrefillArgs& a, int max_groups_in_batch, int nbh,
                               hipStream_t st);
// nbh = entries * hkv (entries = batch in the predicate form, n in the list form).
hipError_t launch_seal_stream(int D, int kb, int vb, const SealStreamArgs& a, int nbh, hipStream_t st);
hipError_t launch_append_seal(int D, int kb, int vb, const AppendSealArgs& a, int nbh, hipStream_t st);
hipError_t launch_append(int D, const CacheArgs& c, const void* k, const void* v, hipStream_t st);
hipError_t launch_prefill_copy(int D, const CacheArgs& c, const void* k, const void* v, int64_t src_tokens,
                               const PrefillLens& lens, int b0, int nb, hipStream_t st);
// phases: 1 = split kernel (partials into the workspace), 2 = combine kernel, 3 = both.
hipError_t launch_decode(int D, int kb, int vb, int gq, const DecodeArgs& a, int phases, hipStream_t st);
hipError_t launch_dequant(int D, int bits, int kind, const void* src, int64_t src_stride, void* dst, int n,
                          hipStream_t st);

#ifdef KVARN_WAVE_TRACE
// Trace build only: copy (host non-NULL) or clear (host NULL) the per-wave
// timestamp buffer of the decode / seal kernels (see trace.hpp).
hipError_t trace_io_decode(void* host, size_t bytes);
hipError_t trace_io_seal(void* host, size_t bytes);
#endif

}  // namespace kvarn
