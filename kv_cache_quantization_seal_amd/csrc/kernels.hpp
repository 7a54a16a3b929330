// Internal launch interface between the C ABI (kvarn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

constexpr int kMaxPrefillBatch = 256;  // requests per prefill launch

struct PrefillLens {
  int32_t len[kMaxPrefillBatch];
};

struct SealPrefillArgs {
  const __half* k;
  const __half* v;
  int64_t src_tokens;
  uint8_t* records;
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
  uint8_t* records;
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

DecodePlan plan_decode(int D, int hq, int hkv, int batch, int max_groups, int resident_wgs);
// Resident split workgroups on the current device for this configuration.
int decode_resident_wgs(int D, int kb, int vb, int gq);

hipError_t launch_seal_tiles(int D, int bits, int kind, const void* src, void* dst, int64_t stride, float* dbg, int n,
                             int iters, hipStream_t st);
hipError_t launch_seal_prefill(int D, int kb, int vb, const SealPrefillArgs& a, int max_groups_in_batch, int nbh,
                               hipStream_t st);
hipError_t launch_seal_stream(int D, int kb, int vb, const SealStreamArgs& a, int nbh, hipStream_t st);
hipError_t launch_append_seal(int D, int kb, int vb, const AppendSealArgs& a, int nbh, hipStream_t st);
hipError_t launch_append(int D, const CacheArgs& c, const void* k, const void* v, hipStream_t st);
hipError_t launch_prefill_copy(int D, const CacheArgs& c, const void* k, const void* v, int64_t src_tokens,
                               const PrefillLens& lens, int b0, int nb, hipStream_t st);
// phases: 1 = split kernel (partials into the workspace), 2 = combine kernel, 3 = both.
hipError_t launch_decode(int D, int kb, int vb, int gq, const DecodeArgs& a, int phases, hipStream_t st);
hipError_t launch_dequant(int D, int bits, int kind, const void* src, int64_t src_stride, void* dst, int n,
                          hipStream_t st);

}  // namespace kvarn
