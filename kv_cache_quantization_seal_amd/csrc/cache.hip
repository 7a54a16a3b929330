// KVarN cache bookkeeping kernels: append one token, prefill copies, and the
// record -> fp16 conversion.
//
// The sink (positions [0,128)) and the in-progress group (the tail) stay exact
// in fp16; a full tail is sealed into a record
// ["KVarN KV Cache: Implementation and Benchmarks" (anbeeld.com), §2.1 "Sink,
// Body, And Tail"].  Records can be converted back to a standard fp16 layout
// for attention paths that do not read them directly (same section).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace kvarn {

// One workgroup per request: read n, copy every KV head's K and V row into
// its slot, then advance seq_len.  Copies move 16-byte chunks.
template <int D>
__global__ __launch_bounds__(256) void append_kernel(CacheArgs c, const uint4* __restrict__ k_new,
                                                     const uint4* __restrict__ v_new) {
  constexpr int CH = D / 8;  // 16-byte chunks per fp16 row
  const int b = blockIdx.x;
  const int n = c.seq_len[b];
  // Capacity 128 + 128*max_groups + 127: the tail may hold all but the last
  // token of a group that has no record slot left.
  const bool full = n < 0 || n >= kSink + kGroup * c.max_groups + kGroup - 1;
  if (!full) {
    const int slot = n < kSink ? n : (n - kSink) % kGroup;
    uint4* dk = reinterpret_cast<uint4*>(n < kSink ? c.sink_k : c.tail_k);
    uint4* dv = reinterpret_cast<uint4*>(n < kSink ? c.sink_v : c.tail_v);
    const int per_kind = c.hkv * CH;
    for (int i = threadIdx.x; i < 2 * per_kind; i += blockDim.x) {
      const int kind = i / per_kind;
      const int r = i % per_kind;
      const int h = r / CH, part = r % CH;
      const int64_t src = ((int64_t)b * c.hkv + h) * CH + part;
      const int64_t dst = (((int64_t)b * c.hkv + h) * kGroup + slot) * CH + part;
      if (kind == 0)
        dk[dst] = k_new[src];
      else
        dv[dst] = v_new[src];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && !full) c.seq_len[b] = n + 1;
}

// One workgroup per (KV head, request, layer): sink and tail copies of a
// prompt, then the request's length.
template <int D>
__global__ __launch_bounds__(256) void prefill_copy_kernel(SealPrefillArgs a) {
  constexpr int CH = D / 8;
  const int h = blockIdx.x;
  const int bl = blockIdx.y;
  const PrefillLayer& L = a.layer[blockIdx.z];
  const int b = a.b0 + bl;
  const int len = a.lens.len[bl];
  const int n_sink = len < kSink ? len : kSink;
  const int n_groups = len > kSink ? (len - kSink) / kGroup : 0;
  const int tail_lo = kSink + kGroup * n_groups;
  const int n_tail = len > kSink ? len - tail_lo : 0;
  const int64_t bh = (int64_t)b * a.hkv + h;
  uint4* sk = reinterpret_cast<uint4*>(L.sink_k) + bh * kGroup * CH;
  uint4* sv = reinterpret_cast<uint4*>(L.sink_v) + bh * kGroup * CH;
  uint4* tk = reinterpret_cast<uint4*>(L.tail_k) + bh * kGroup * CH;
  uint4* tv = reinterpret_cast<uint4*>(L.tail_v) + bh * kGroup * CH;
  const uint4* ks = reinterpret_cast<const uint4*>(L.k) + bh * a.src_tokens * CH;
  const uint4* vs = reinterpret_cast<const uint4*>(L.v) + bh * a.src_tokens * CH;
  for (int i = threadIdx.x; i < n_sink * CH; i += blockDim.x) {
    sk[i] = ks[i];
    sv[i] = vs[i];
  }
  for (int i = threadIdx.x; i < n_tail * CH; i += blockDim.x) {
    tk[i] = ks[(int64_t)tail_lo * CH + i];
    tv[i] = vs[(int64_t)tail_lo * CH + i];
  }
  if (h == 0 && threadIdx.x == 0) L.seq_len[b] = len;
}

// Record -> fp16 original-frame rows.  The record is staged in LDS with
// 16-byte loads; thread (token t, 32-channel block bl), NB = D/32 threads per
// token, rebuilds s_t (code - mid) c_j for its 32 channels, rotates by
// H_D / sqrt(D) (butterflies over the five low channel bits in registers,
// over the block bits across neighbouring lanes), and writes its 64 bytes.
// A row of codes is a little-endian bit stream: code i occupies bits
// [BITS i, BITS i + BITS).
template <int M>
__device__ __forceinline__ float dq_pair(float x) {
  const int v = __float_as_int(x);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true));
  else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true));
  else {
    const int o = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);  // lanes 0-3 <- 4-7
    return __int_as_float(__builtin_amdgcn_update_dpp(o, v, 0x114, 0xF, 0xA, false));  // 4-7 <- 0-3
  }
}

template <int D, int BITS, int KIND>
__global__ __launch_bounds__(4 * D) void dequant_kernel(const uint8_t* __restrict__ src, int64_t src_stride,
                                                        __half* __restrict__ dst) {
  constexpr int NB = D / 32;
  constexpr int CODE_BYTES = kGroup * D * BITS / 8;
  constexpr int REC = CODE_BYTES + 2 * kGroup + 2 * D;  // a multiple of 16
  constexpr float MID = 0.5f * ((1 << BITS) - 1);
  constexpr int ROWBITS = (KIND == 0 ? D : kGroup) * BITS;
  __shared__ uint32_t rs_[REC / 4];
  const uint8_t* rec = src + blockIdx.x * src_stride;
  for (int i = threadIdx.x; i < REC / 16; i += blockDim.x)
    reinterpret_cast<uint4*>(rs_)[i] = reinterpret_cast<const uint4*>(rec)[i];
  __syncthreads();
  const uint16_t* s16 = reinterpret_cast<const uint16_t*>(rs_) + CODE_BYTES / 2;
  const uint16_t* c16 = s16 + kGroup;
  const int t = threadIdx.x / NB, bl = threadIdx.x % NB;
  const float st = h2f(s16[t]);
  float x[32];
  uint32_t code[32];
  if constexpr (KIND == 0) {
    // Token t's codes 32 bl .. 32 bl + 31 are BITS consecutive dwords of
    // its row (row and run starts are multiples of 32 bits): load them once,
    // then one bit-field extract (or funnel shift) per code at a fixed place.
    const uint32_t* w = rs_ + (t * ROWBITS + 32 * BITS * bl) / 32;
    uint32_t r[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) r[k] = w[k];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int b0 = BITS * i, k = b0 / 32, sh = b0 % 32;
      if (sh + BITS <= 32)
        code[i] = __builtin_amdgcn_ubfe(r[k], sh, BITS);
      else
        code[i] = __builtin_amdgcn_alignbit(r[k + 1], r[k], sh) & ((1u << BITS) - 1);
    }
  } else {
    // Channel rows: channel j's code of token t sits at the same place in
    // every row (bit BITS t), rows 4 BITS dwords apart.  A code that crosses
    // into the next dword (odd widths) reads it too; that dword is still in
    // the record (the scales follow the codes).
    const int dw = (BITS * t) >> 5, sh = (BITS * t) & 31;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t* w = rs_ + (32 * bl + i) * (ROWBITS / 32) + dw;
      if constexpr (32 % BITS == 0)
        code[i] = __builtin_amdgcn_ubfe(w[0], sh, BITS);
      else
        code[i] = __builtin_amdgcn_alignbit(w[1], w[0], sh) & ((1u << BITS) - 1);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = st * ((float)code[i] - MID) * h2f(c16[32 * bl + i]);
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & s)) {
        const float a0 = x[i], a1 = x[i + s];
        x[i] = a0 + a1;
        x[i + s] = a0 - a1;
      }
    }
  }
  // Block bits: the lane with the bit set keeps x - x' negated (x + s x',
  // s = -1); the negations commute with later stages and the final sign
  // undoes them.
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fmaf((bl & 1) ? -1.0f : 1.0f, dq_pair<1>(x[i]), x[i]);
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = fmaf((bl & 2) ? -1.0f : 1.0f, dq_pair<2>(x[i]), x[i]);
  if constexpr (NB == 8) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = fmaf((bl & 4) ? -1.0f : 1.0f, dq_pair<4>(x[i]), x[i]);
  }
  const float rs = ((D == 128) ? 0.08838834764831845f : 0.0625f) * ((__popc(bl) & 1) ? -1.0f : 1.0f);
  // Through LDS, so that each store instruction writes consecutive 16-byte
  // pieces across the lanes (a lane's own 64 bytes leave 48-byte gaps between
  // lanes); 8192 2-bit records at D 128: 98 -> 68 us, V records at D 256:
  // 197 -> 178 us.  For K records at D 256 (a 64 KB tile) the staged form was
  // slower (202 -> 248 us), so there the lanes store their own 64 bytes.
  if constexpr (D == 128 || KIND == 1) {
    __shared__ uint4 os_[kGroup * D / 8];  // the fp16 output tile, row-major
    uint4* orow = os_ + (t * D + 32 * bl) / 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t wd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wd[e] = (uint32_t)f2h_rne(x[8 * k + 2 * e] * rs) | ((uint32_t)f2h_rne(x[8 * k + 2 * e + 1] * rs) << 16);
      orow[k] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    lds_barrier();
    uint4* out = reinterpret_cast<uint4*>(dst + (int64_t)blockIdx.x * kGroup * D);
    if constexpr (D == 128) {
      // Streaming (nontemporal) stores: the tile is written once and not read
      // back here.  8192 records at D 128: 67-79 -> 62-66 us; at D 256 (64 KB
      // tiles) they were slower (V records 186 -> 248 us), so not used there.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 o = os_[threadIdx.x + 4 * D * k];
        __builtin_nontemporal_store(v4i{(int)o.x, (int)o.y, (int)o.z, (int)o.w},
                                    reinterpret_cast<v4i*>(out + threadIdx.x + 4 * D * k));
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[threadIdx.x + 4 * D * k] = os_[threadIdx.x + 4 * D * k];
    }
  } else {
    uint4* out = reinterpret_cast<uint4*>(dst + ((int64_t)blockIdx.x * kGroup + t) * D + 32 * bl);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t wd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wd[e] = (uint32_t)f2h_rne(x[8 * k + 2 * e] * rs) | ((uint32_t)f2h_rne(x[8 * k + 2 * e + 1] * rs) << 16);
      out[k] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
  }
}

hipError_t launch_append(int D, const CacheArgs& c, const void* k, const void* v, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL(append_kernel<128>, dim3(c.batch), dim3(256), 0, st, c, (const uint4*)k, (const uint4*)v);
  else
    hipLaunchKernelGGL(append_kernel<256>, dim3(c.batch), dim3(256), 0, st, c, (const uint4*)k, (const uint4*)v);
  return hipGetLastError();
}

hipError_t launch_prefill_copy(int D, const SealPrefillArgs& a, int nb, hipStream_t st) {
  if (nb <= 0 || a.n_layers <= 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(prefill_copy_kernel<128>, dim3(a.hkv, nb, a.n_layers), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(prefill_copy_kernel<256>, dim3(a.hkv, nb, a.n_layers), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int BITS>
static void launch_dq(int kind, const void* src, int64_t stride, void* dst, int n, hipStream_t st) {
  if (kind == 0)
    hipLaunchKernelGGL((dequant_kernel<D, BITS, 0>), dim3(n), dim3(4 * D), 0, st, (const uint8_t*)src, stride,
                       (__half*)dst);
  else
    hipLaunchKernelGGL((dequant_kernel<D, BITS, 1>), dim3(n), dim3(4 * D), 0, st, (const uint8_t*)src, stride,
                       (__half*)dst);
}

hipError_t launch_dequant(int D, int bits, int kind, const void* src, int64_t src_stride, void* dst, int n,
                          hipStream_t st) {
#define CALL(d, b) launch_dq<d, b>(kind, src, src_stride, dst, n, st)
  KVARN_DISPATCH_DB(D, bits, CALL);
#undef CALL
  return hipGetLastError();
}

}  // namespace kvarn
