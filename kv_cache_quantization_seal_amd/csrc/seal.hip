// KVarN group sealing on gfx950.
//
// One workgroup seals one 128 x D tile (one KV head, one group, K or V):
//   1. Hadamard rotation along channels (natural-order Sylvester H_D / sqrt(D))
//      [P1 "What it is"; P2 §1 "Where KVarN Comes From"];
//   2. `iters` Sinkhorn-style iterations, each rescaling every token row and
//      then every channel column to unit mean square [P1 "What it is"; P2 §1:
//      16 iterations];
//   3. per-token round to nearest on a symmetric mid-rise grid whose step
//      comes from the token's largest normalized magnitude, codes packed with
//      fp16 token scales s_t and channel scales c_j [P1 "What it is";
//      P2 §2.1: the record keeps the payload with its scale metadata].
// P1 = "KVarN: Variance-Normalized KV-Cache Quantization Mitigates Error
// Accumulation in Reasoning Tasks" (fig1.dev summary); P2 = "KVarN KV Cache:
// Implementation and Benchmarks" (anbeeld.com).
//
// Factor form of the Sinkhorn step.  With A = X_r * X_r (elementwise) and
// running factors r, c, the row step of the literal rescaling gives
// r_t^2 = mean_j A_tj / c_j^2 and the column step c_j^2 = mean_t A_tj / r_t^2
// (each new factor is independent of its own previous value), so one
// iteration is two matrix-vector products with u = 1/c^2 and v = 1/r^2.  A row
// or column whose mean square is zero keeps its factor.  The final record only
// needs c and X_r: s_t = 2 max_j |X_r,tj / c_j| / (2^b - 1) and
// code = rne(X_r,tj / c_j / s_t + mid).
//
// Data layout in the workgroup (2*D threads, D/32 waves):
//   row role: wave w owns token t = 64*(w / (D/64)) + lane and the 64 channels
//             of block w % (D/64)  -> A_row[64] in VGPRs;
//   col role: wave w owns channel j = 64*(w / 2) + lane and the 64 tokens of
//             half w % 2             -> A_col[64] in VGPRs;
//   LDS holds X_r (fp32, row pitch D+4) plus the factor vectors.  Each
//   half-step is 64 register FMAs per thread against an LDS-broadcast vector,
//   a partial-sum exchange and one owner-computed division.
#include "common.hpp"
#include "kernels.hpp"

namespace kvarn {

template <int D>
struct SealSmem {
  static constexpr int kPitch = D + 4;
  static constexpr int kBlocks = D / 64;
  float x[kGroup * kPitch];
  float u[D];                 // 1 / c_j^2
  float v[kGroup];            // 1 / r_t^2
  float part[kBlocks][kGroup];  // row partials (sums, then maxima)
  float qcol[2][D];           // column partials
  float c2[D];                // c_j^2
  float cinv[D];              // 1 / c_j
  float inv[kGroup];          // per-token inverse step (2^b - 1) / (2 M_t)
};

template <int D, int BITS, bool TOKEN_MAJOR>
__device__ __forceinline__ void seal_body(const __half* __restrict__ src, uint8_t* __restrict__ rec,
                                          float* __restrict__ dbg, int iters, SealSmem<D>& sm) {
  constexpr int NB = D / 64;
  constexpr int P = SealSmem<D>::kPitch;
  constexpr int LEVELS = (1 << BITS) - 1;
  constexpr float MID = 0.5f * LEVELS;
  constexpr int CODE_BYTES = kGroup * D * BITS / 8;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int rb = w % NB;            // row role: channel block
  const int t = 64 * (w / NB) + lane;  // row role: token
  const int ca = w & 1;             // col role: token half
  const int j = 64 * (w >> 1) + lane;  // col role: channel

  float x[64];
  {
    const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)t * D + 64 * rb);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 q = p[k];
      const uint32_t ws[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * k + 2 * e] = h2f((uint16_t)(ws[e] & 0xFFFFu));
        x[8 * k + 2 * e + 1] = h2f((uint16_t)(ws[e] >> 16));
      }
    }
  }
  float* xrow = sm.x + t * P + 64 * rb;
  rotate_row_slice<D, P>(x, sm.x, t, rb);
  const float rs = (D == 128) ? 0.08838834764831845f : 0.0625f;  // 1/sqrt(D)
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] *= rs;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    *reinterpret_cast<float4*>(xrow + 4 * k) = make_float4(x[4 * k], x[4 * k + 1], x[4 * k + 2], x[4 * k + 3]);
  // x now becomes A_row = X_r^2.
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] *= x[i];
  if (ca == 0) {
    sm.u[j] = 1.0f;
    sm.c2[j] = 1.0f;
  }
  __syncthreads();
  float acol[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const float a = sm.x[(64 * ca + i) * P + j];
    acol[i] = a * a;
  }

  for (int it = 0; it < iters; ++it) {
    // Token step: r_t^2 = mean_j A_tj u_j.
    {
      float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
      const float* ub = sm.u + 64 * rb;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(ub + 4 * k);
        p0 = fmaf(x[4 * k], q.x, p0);
        p1 = fmaf(x[4 * k + 1], q.y, p1);
        p2 = fmaf(x[4 * k + 2], q.z, p2);
        p3 = fmaf(x[4 * k + 3], q.w, p3);
      }
      sm.part[rb][t] = (p0 + p1) + (p2 + p3);
    }
    __syncthreads();
    if (rb == 0) {
      float tot = sm.part[0][t];
#pragma unroll
      for (int o = 1; o < NB; ++o) tot += sm.part[o][t];
      sm.v[t] = tot > 0.f ? (float)D / tot : 0.f;
    }
    __syncthreads();
    // Channel step: c_j^2 = mean_t A_tj v_t.
    {
      float q0 = 0.f, q1 = 0.f, q2 = 0.f, q3 = 0.f;
      const float* vb = sm.v + 64 * ca;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(vb + 4 * k);
        q0 = fmaf(acol[4 * k], q.x, q0);
        q1 = fmaf(acol[4 * k + 1], q.y, q1);
        q2 = fmaf(acol[4 * k + 2], q.z, q2);
        q3 = fmaf(acol[4 * k + 3], q.w, q3);
      }
      sm.qcol[ca][j] = (q0 + q1) + (q2 + q3);
    }
    __syncthreads();
    if (ca == 0) {
      const float tot = sm.qcol[0][j] + sm.qcol[1][j];
      if (tot > 0.f) {
        sm.c2[j] = tot * (1.0f / kGroup);
        sm.u[j] = (float)kGroup / tot;
      } else {
        sm.u[j] = 0.f;
      }
    }
    __syncthreads();
  }

  // Channel scales.
  if (ca == 0) {
    const float c = sqrtf(sm.c2[j]);
    sm.cinv[j] = 1.0f / c;
    reinterpret_cast<uint16_t*>(rec + CODE_BYTES + 2 * kGroup)[j] = f2h_rne(c);
    if (dbg) dbg[kGroup + j] = c;
  }
  __syncthreads();
  // Token scales from the largest |X_r / c| of each token.
  float z[64];
  float mx = 0.f;
  {
    const float* cb = sm.cinv + 64 * rb;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(xrow + 4 * k);
      const float4 ci = *reinterpret_cast<const float4*>(cb + 4 * k);
      z[4 * k] = a.x * ci.x;
      z[4 * k + 1] = a.y * ci.y;
      z[4 * k + 2] = a.z * ci.z;
      z[4 * k + 3] = a.w * ci.w;
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) mx = fmaxf(mx, fabsf(z[i]));
  }
  if constexpr (NB > 1) {
    sm.part[rb][t] = mx;
    __syncthreads();
#pragma unroll
    for (int o = 0; o < NB; ++o) mx = fmaxf(mx, sm.part[o][t]);
  }
  const float inv = mx > 0.f ? (float)LEVELS / (2.0f * mx) : 0.f;
  if (rb == 0) {
    const float s = mx * (2.0f / LEVELS);
    reinterpret_cast<uint16_t*>(rec + CODE_BYTES)[t] = f2h_rne(s);
    if (dbg) dbg[t] = s;
    sm.inv[t] = inv;
  }
  if constexpr (TOKEN_MAJOR) {
    // K record: token t's codes for channels [64 rb, 64 rb + 64).
    constexpr int WORDS = 64 * BITS / 32;
    constexpr int PER = 32 / BITS;
    uint32_t out[WORDS];
#pragma unroll
    for (int k = 0; k < WORDS; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float c = fminf(fmaxf(rintf(fmaf(z[k * PER + e], inv, MID)), 0.f), (float)LEVELS);
        word |= (uint32_t)c << (BITS * e);
      }
      out[k] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(rec + (size_t)t * (D * BITS / 8) + rb * (64 * BITS / 8));
#pragma unroll
    for (int k = 0; k < WORDS / 4; ++k) dst[k] = make_uint4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
  } else {
    // V record: channel j's codes for tokens [64 ca, 64 ca + 64).
    __syncthreads();
    constexpr int WORDS = 64 * BITS / 32;
    constexpr int PER = 32 / BITS;
    const float ci = sm.cinv[j];
    uint32_t out[WORDS];
#pragma unroll
    for (int k = 0; k < WORDS; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int tok = 64 * ca + k * PER + e;
        const float zz = sm.x[tok * P + j] * ci;
        const float c = fminf(fmaxf(rintf(fmaf(zz, sm.inv[tok], MID)), 0.f), (float)LEVELS);
        word |= (uint32_t)c << (BITS * e);
      }
      out[k] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(rec + (size_t)j * (kGroup * BITS / 8) + ca * (64 * BITS / 8));
#pragma unroll
    for (int k = 0; k < WORDS / 4; ++k) dst[k] = make_uint4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
template <int D, int BITS, int KIND>
__global__ __launch_bounds__(2 * D) void seal_tiles_kernel(const __half* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int64_t dst_stride, float* __restrict__ dbg, int iters) {
  __shared__ SealSmem<D> sm;
  const int64_t i = blockIdx.x;
  seal_body<D, BITS, KIND == 0>(src + i * kGroup * D, dst + i * dst_stride, dbg ? dbg + i * (kGroup + D) : nullptr,
                                iters, sm);
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(2 * D) void seal_prefill_kernel(SealPrefillArgs a) {
  __shared__ SealSmem<D> sm;
  const int g = blockIdx.x;
  const int bl = blockIdx.y / a.hkv, h = blockIdx.y % a.hkv;
  const int kind = blockIdx.z;
  const int len = a.lens.len[bl];
  if (kSink + kGroup * (g + 1) > len) return;
  const int64_t bh = (int64_t)(a.b0 + bl) * a.hkv + h;
  const __half* src = (kind ? a.v : a.k) + (bh * a.src_tokens + kSink + (int64_t)kGroup * g) * D;
  uint8_t* rec = a.records + (bh * a.max_groups + g) * a.group_bytes + (kind ? a.rec_k_bytes : 0);
  if (kind == 0)
    seal_body<D, KB, true>(src, rec, nullptr, a.iters, sm);
  else
    seal_body<D, VB, false>(src, rec, nullptr, a.iters, sm);
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(2 * D) void seal_stream_kernel(SealStreamArgs a) {
  __shared__ SealSmem<D> sm;
  const int bh = blockIdx.x;
  const int kind = blockIdx.y;
  const int b = bh / a.hkv;
  const int n = a.seq_len[b];
  if (n < kSink + kGroup || ((n - kSink) % kGroup) != 0) return;
  const int g = (n - kSink) / kGroup - 1;
  if (g >= a.max_groups) return;
  const __half* src = (kind ? a.tail_v : a.tail_k) + (int64_t)bh * kGroup * D;
  uint8_t* rec = a.records + ((int64_t)bh * a.max_groups + g) * a.group_bytes + (kind ? a.rec_k_bytes : 0);
  if (kind == 0)
    seal_body<D, KB, true>(src, rec, nullptr, a.iters, sm);
  else
    seal_body<D, VB, false>(src, rec, nullptr, a.iters, sm);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int BITS>
static hipError_t launch_tiles_db(int kind, const void* src, void* dst, int64_t stride, float* dbg, int n, int iters,
                                  hipStream_t st) {
  if (kind == 0)
    hipLaunchKernelGGL((seal_tiles_kernel<D, BITS, 0>), dim3(n), dim3(2 * D), 0, st, (const __half*)src,
                       (uint8_t*)dst, stride, dbg, iters);
  else
    hipLaunchKernelGGL((seal_tiles_kernel<D, BITS, 1>), dim3(n), dim3(2 * D), 0, st, (const __half*)src,
                       (uint8_t*)dst, stride, dbg, iters);
  return hipGetLastError();
}

hipError_t launch_seal_tiles(int D, int bits, int kind, const void* src, void* dst, int64_t stride, float* dbg, int n,
                             int iters, hipStream_t st) {
  if (D == 128) return bits == 2 ? launch_tiles_db<128, 2>(kind, src, dst, stride, dbg, n, iters, st)
                                 : launch_tiles_db<128, 4>(kind, src, dst, stride, dbg, n, iters, st);
  return bits == 2 ? launch_tiles_db<256, 2>(kind, src, dst, stride, dbg, n, iters, st)
                   : launch_tiles_db<256, 4>(kind, src, dst, stride, dbg, n, iters, st);
}

template <int D, int KB, int VB>
static void launch_prefill_t(const SealPrefillArgs& a, int gx, int gy, hipStream_t st) {
  hipLaunchKernelGGL((seal_prefill_kernel<D, KB, VB>), dim3(gx, gy, 2), dim3(2 * D), 0, st, a);
}
template <int D, int KB, int VB>
static void launch_stream_t(const SealStreamArgs& a, int gx, hipStream_t st) {
  hipLaunchKernelGGL((seal_stream_kernel<D, KB, VB>), dim3(gx, 2), dim3(2 * D), 0, st, a);
}

#define KVARN_DISPATCH_DKV(D, KB, VB, CALL)                       \
  do {                                                            \
    if (D == 128) {                                               \
      if (KB == 2 && VB == 2) CALL(128, 2, 2);                    \
      else if (KB == 2 && VB == 4) CALL(128, 2, 4);               \
      else if (KB == 4 && VB == 2) CALL(128, 4, 2);               \
      else CALL(128, 4, 4);                                       \
    } else {                                                      \
      if (KB == 2 && VB == 2) CALL(256, 2, 2);                    \
      else if (KB == 2 && VB == 4) CALL(256, 2, 4);               \
      else if (KB == 4 && VB == 2) CALL(256, 4, 2);               \
      else CALL(256, 4, 4);                                       \
    }                                                             \
  } while (0)

hipError_t launch_seal_prefill(int D, int kb, int vb, const SealPrefillArgs& a, int max_groups_in_batch, int nbh,
                               hipStream_t st) {
  if (max_groups_in_batch <= 0 || nbh <= 0) return hipSuccess;
#define CALL(d, k, v) launch_prefill_t<d, k, v>(a, max_groups_in_batch, nbh, st)
  KVARN_DISPATCH_DKV(D, kb, vb, CALL);
#undef CALL
  return hipGetLastError();
}

hipError_t launch_seal_stream(int D, int kb, int vb, const SealStreamArgs& a, int nbh, hipStream_t st) {
  if (nbh <= 0) return hipSuccess;
#define CALL(d, k, v) launch_stream_t<d, k, v>(a, nbh, st)
  KVARN_DISPATCH_DKV(D, kb, vb, CALL);
#undef CALL
  return hipGetLastError();
}

}  // namespace kvarn
