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
// Data layout in the workgroup (2*D threads, D/32 waves), after the rotation:
//   row role: lane l of wave w owns tokens 4*tq .. 4*tq+3 and channels
//             16*cb .. 16*cb+15 (tq = RPW*w + l / RL, cb = l % RL, RL = D/16
//             lanes per token quad) -> A_row[4][16] in VGPRs;
//   col role: lane l of wave w owns channels 4*cq .. 4*cq+3 and tokens
//             16*tb .. 16*tb+15 (cq = 8*w + l / 8, tb = l % 8)
//             -> A_col[16][4] in VGPRs.
//   LDS holds X_r (fp32, row pitch D+4) plus the factor vectors.  A half-step
//   reads 16 factors from LDS (four 128-bit broadcasts) for 64 register FMAs;
//   the partial sums of a token quad (channel quad) sit in RL (8) adjacent
//   lanes and meet through DPP; the first lane publishes the four new
//   factors.  One barrier per half-step.
#include "common.hpp"
#include "kernels.hpp"

namespace kvarn {

template <int D>
struct alignas(16) SealSmem {
  static constexpr int kPitch = D + 4;
  static constexpr int kBlocks = D / 64;
  float x[kGroup * kPitch];
  float u[D];                 // 1 / c_j^2
  float v[kGroup];            // 1 / r_t^2
  float c2[D];                // c_j^2
  float cinv[D];              // 1 / c_j
  float inv[kGroup];          // per-token inverse step (2^b - 1) / (2 M_t)
};

// Sum / maximum over the 8 lanes 8k .. 8k+7 (every lane receives it).
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  return v;
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return v;
}
template <int RL>
__device__ __forceinline__ float sum_rl(float v) {
  return RL == 8 ? sum8(v) : row16_sum(v);
}
template <int RL>
__device__ __forceinline__ float max_rl(float v) {
  return RL == 8 ? max8(v) : row16_max(v);
}

template <int D, int BITS, bool TOKEN_MAJOR>
__device__ __forceinline__ void seal_body(const __half* __restrict__ src, uint8_t* __restrict__ rec,
                                          float* __restrict__ dbg, int iters, SealSmem<D>& sm) {
  constexpr int NB = D / 64;
  constexpr int P = SealSmem<D>::kPitch;
  constexpr int LEVELS = (1 << BITS) - 1;
  constexpr float MID = 0.5f * LEVELS;
  constexpr int CODE_BYTES = kGroup * D * BITS / 8;
  constexpr int RL = D / 16;          // row role: lanes per token quad
  constexpr int RPW = 64 / RL;        // row role: token quads per wave
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;

  // ---- rotation: thread (token tl, 64-channel block bl) ------------------
  {
    const int bl = w % NB;
    const int tl = 64 * (w / NB) + lane;
    float x[64];
    const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)tl * D + 64 * bl);
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
    rotate_row_slice<D, P>(x, sm.x, tl, bl);
    const float rs = (D == 128) ? 0.08838834764831845f : 0.0625f;  // 1/sqrt(D)
    float* xrow = sm.x + tl * P + 64 * bl;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      *reinterpret_cast<float4*>(xrow + 4 * k) =
          make_float4(x[4 * k] * rs, x[4 * k + 1] * rs, x[4 * k + 2] * rs, x[4 * k + 3] * rs);
  }
  if (tid < D) {
    sm.u[tid] = 1.0f;
    sm.c2[tid] = 1.0f;
  }
  __syncthreads();

  // ---- A = X_r^2 blocks --------------------------------------------------
  const int tq = RPW * w + lane / RL, cb = lane % RL;  // row role
  const int cq = 8 * w + (lane >> 3), tb = lane & 7;   // col role
  float ar[4][16], ac[16][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float* xr = sm.x + (4 * tq + r) * P + 16 * cb;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(xr + 4 * k);
      ar[r][4 * k] = a.x * a.x;
      ar[r][4 * k + 1] = a.y * a.y;
      ar[r][4 * k + 2] = a.z * a.z;
      ar[r][4 * k + 3] = a.w * a.w;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 a = *reinterpret_cast<const float4*>(sm.x + (16 * tb + i) * P + 4 * cq);
    ac[i][0] = a.x * a.x;
    ac[i][1] = a.y * a.y;
    ac[i][2] = a.z * a.z;
    ac[i][3] = a.w * a.w;
  }

  for (int it = 0; it < iters; ++it) {
    // Token step: r_t^2 = mean_j A_tj u_j.
    {
      float uv[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(sm.u + 16 * cb + 4 * k);
        uv[4 * k] = q.x;
        uv[4 * k + 1] = q.y;
        uv[4 * k + 2] = q.z;
        uv[4 * k + 3] = q.w;
      }
      float tot[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int c = 0; c < 16; c += 2) {
          p0 = fmaf(ar[r][c], uv[c], p0);
          p1 = fmaf(ar[r][c + 1], uv[c + 1], p1);
        }
        tot[r] = sum_rl<RL>(p0 + p1);
      }
      if (cb == 0) {
        float4 vv;
        vv.x = tot[0] > 0.f ? (float)D * __builtin_amdgcn_rcpf(tot[0]) : 0.f;
        vv.y = tot[1] > 0.f ? (float)D * __builtin_amdgcn_rcpf(tot[1]) : 0.f;
        vv.z = tot[2] > 0.f ? (float)D * __builtin_amdgcn_rcpf(tot[2]) : 0.f;
        vv.w = tot[3] > 0.f ? (float)D * __builtin_amdgcn_rcpf(tot[3]) : 0.f;
        *reinterpret_cast<float4*>(sm.v + 4 * tq) = vv;
      }
    }
    __syncthreads();
    // Channel step: c_j^2 = mean_t A_tj v_t.
    {
      float vt[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(sm.v + 16 * tb + 4 * k);
        vt[4 * k] = q.x;
        vt[4 * k + 1] = q.y;
        vt[4 * k + 2] = q.z;
        vt[4 * k + 3] = q.w;
      }
      float tot[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float q0 = 0.f, q1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          q0 = fmaf(ac[i][c], vt[i], q0);
          q1 = fmaf(ac[i + 1][c], vt[i + 1], q1);
        }
        tot[c] = sum8(q0 + q1);
      }
      if (tb == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (tot[c] > 0.f) {
            sm.c2[4 * cq + c] = tot[c] * (1.0f / kGroup);
            sm.u[4 * cq + c] = (float)kGroup * __builtin_amdgcn_rcpf(tot[c]);
          } else {
            sm.u[4 * cq + c] = 0.f;
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- channel scales ----------------------------------------------------
  if (tid < D) {
    const float c = sqrtf(sm.c2[tid]);
    sm.cinv[tid] = 1.0f / c;
    reinterpret_cast<uint16_t*>(rec + CODE_BYTES + 2 * kGroup)[tid] = f2h_rne(c);
    if (dbg) dbg[kGroup + tid] = c;
  }
  __syncthreads();

  // ---- token scales from the largest |X_r / c| of each token (row role) ---
  float zr[4][16];
  float inv[4];
  {
    float ci[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 q = *reinterpret_cast<const float4*>(sm.cinv + 16 * cb + 4 * k);
      ci[4 * k] = q.x;
      ci[4 * k + 1] = q.y;
      ci[4 * k + 2] = q.z;
      ci[4 * k + 3] = q.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float* xr = sm.x + (4 * tq + r) * P + 16 * cb;
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(xr + 4 * k);
        zr[r][4 * k] = a.x * ci[4 * k];
        zr[r][4 * k + 1] = a.y * ci[4 * k + 1];
        zr[r][4 * k + 2] = a.z * ci[4 * k + 2];
        zr[r][4 * k + 3] = a.w * ci[4 * k + 3];
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) mx = fmaxf(mx, fabsf(zr[r][c]));
      mx = max_rl<RL>(mx);
      inv[r] = mx > 0.f ? (float)LEVELS / (2.0f * mx) : 0.f;
      if (cb == 0) {
        const int t = 4 * tq + r;
        const float sc = mx * (2.0f / LEVELS);
        reinterpret_cast<uint16_t*>(rec + CODE_BYTES)[t] = f2h_rne(sc);
        if (dbg) dbg[t] = sc;
        sm.inv[t] = inv[r];
      }
    }
  }
  if constexpr (TOKEN_MAJOR) {
    // K record: tokens 4tq .. 4tq+3, channels [16 cb, 16 cb + 16): one
    // (2-bit) or two (4-bit) little-endian words per token.
    constexpr int WORDS = 16 * BITS / 32;
    constexpr int PER = 32 / BITS;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint32_t out[WORDS];
#pragma unroll
      for (int k = 0; k < WORDS; ++k) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const float c = fminf(fmaxf(rintf(fmaf(zr[r][k * PER + e], inv[r], MID)), 0.f), (float)LEVELS);
          word |= (uint32_t)c << (BITS * e);
        }
        out[k] = word;
      }
      uint8_t* dst = rec + (size_t)(4 * tq + r) * (D * BITS / 8) + cb * (16 * BITS / 8);
      if constexpr (WORDS == 1)
        *reinterpret_cast<uint32_t*>(dst) = out[0];
      else
        *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
    }
  } else {
    // V record: channels 4cq .. 4cq+3, tokens [16 tb, 16 tb + 16).
    __syncthreads();
    constexpr int WORDS = 16 * BITS / 32;
    constexpr int PER = 32 / BITS;
    const float4 ci = *reinterpret_cast<const float4*>(sm.cinv + 4 * cq);
    float zc[16][4], iv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(sm.x + (16 * tb + i) * P + 4 * cq);
      zc[i][0] = a.x * ci.x;
      zc[i][1] = a.y * ci.y;
      zc[i][2] = a.z * ci.z;
      zc[i][3] = a.w * ci.w;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 q = *reinterpret_cast<const float4*>(sm.inv + 16 * tb + 4 * k);
      iv[4 * k] = q.x;
      iv[4 * k + 1] = q.y;
      iv[4 * k + 2] = q.z;
      iv[4 * k + 3] = q.w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t out[WORDS];
#pragma unroll
      for (int k = 0; k < WORDS; ++k) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int i = k * PER + e;
          const float code = fminf(fmaxf(rintf(fmaf(zc[i][c], iv[i], MID)), 0.f), (float)LEVELS);
          word |= (uint32_t)code << (BITS * e);
        }
        out[k] = word;
      }
      uint8_t* dst = rec + (size_t)(4 * cq + c) * (kGroup * BITS / 8) + tb * (16 * BITS / 8);
      if constexpr (WORDS == 1)
        *reinterpret_cast<uint32_t*>(dst) = out[0];
      else
        *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
    }
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
