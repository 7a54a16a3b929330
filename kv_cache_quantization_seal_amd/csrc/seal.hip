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
// Data layout in the workgroup (4*D threads, D/16 waves):
//   rotation: thread (token tid / NB, 32-channel block tid % NB), NB = D/32,
//             loads its 64 bytes of the fp16 tile; butterflies over the five
//             low channel bits run in registers, over the block bits across
//             neighbouring lanes (DPP); X_r goes to LDS (fp32, row pitch D+4,
//             16-byte groups swizzled so that every 128-bit access pattern
//             below is free of bank conflicts).
//   row role: lane l of wave w owns tokens 2*tp, 2*tp+1 and channels
//             16*cb .. 16*cb+15 (tp = RPW*w + l / RL, cb = l % RL, RL = D/16
//             lanes per token pair) -> A_row[2][16] in VGPRs;
//   col role: lane l of wave w owns channels 2*cp, 2*cp+1 and tokens
//             16*tb .. 16*tb+15 (cp = 8*w + l / 8, tb = l % 8)
//             -> A_col[16][2] in VGPRs.
//   A half-step reads 16 factors from LDS (four 128-bit reads of a skewed
//   vector) for 32 register FMAs; the partial sums of a token pair (channel
//   pair) sit in RL (8) adjacent lanes and meet through DPP; the first two
//   lanes publish the two new factors.  One barrier per half-step.  About 110
//   VGPRs per lane and 70 KB (D 128) of LDS give two workgroups, four waves
//   per SIMD, on a CU.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace kvarn {

// Threads per workgroup = kSealThreadsPerD * D (one 128 x D tile).
constexpr int kSealThreadsPerD = 4;

// Factor vectors are stored skewed, element j at sk(j) = j + 4 (j >> 4):
// sixteen-element runs start 20 dwords apart, so the eight lanes that read
// runs 0..7 with one 128-bit access each hit eight different bank quads.
__device__ __forceinline__ constexpr int sk(int j) { return j + 4 * (j >> 4); }

template <int D>
struct alignas(16) SealSmem {
  static constexpr int kPitch = D + 4;
  static constexpr int kBlocks = D / 64;
  float x[kGroup * kPitch];    // X_r, 16-byte groups at xgrp positions
  float u[D + D / 4];          // 1 / c_j^2 (skewed)
  float v[kGroup + kGroup / 4];  // 1 / r_t^2 (skewed)
  float c2[D];                 // c_j^2
  float cinv[D + D / 4];       // 1 / c_j (skewed)
  float inv[kGroup + kGroup / 4];  // per-token inverse step (2^b - 1) / (2 M_t) (skewed)
};

// Address of 16-byte group g of row t of the X_r tile.
template <int D>
__device__ __forceinline__ float* xg(SealSmem<D>& sm, int t, int g) {
  return sm.x + t * SealSmem<D>::kPitch + 4 * xgrp(g, t);
}

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

// Rotation layout.  Thread (token tid / NB, block bl = tid % NB), NB = D / 32,
// loads channels 32 bl .. 32 bl + 31 of its token; block bit m of bl is paired
// with register bit q_m = 4 - m (value i of the block sits in register slot
// i ^ relabel(bl), relabel(bl) = sum over set bits m of 2^q_m), so that the
// lane stages below can exchange half of the values each.
template <int D>
__device__ __forceinline__ int rot_relabel(int bl) {
  return ((bl & 1) << 4) | ((bl & 2) << 2) | (D == 256 ? (bl & 4) : 0);
}

// The thread's 64 bytes of the fp16 tile in register-slot order: slots
// 8k .. 8k+7 in raw[k].
template <int D>
__device__ __forceinline__ void load_tile(uint4 (&raw)[4], const __half* __restrict__ src, int tid) {
  constexpr int NB = D / 32;
  const int bl = tid % NB;
  const __half* base = src + (size_t)(tid / NB) * D + 32 * bl;
  const int pk = rot_relabel<D>(bl) >> 3;  // 16-byte piece swap (slot bits 3, 4)
  if constexpr (NB == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = reinterpret_cast<const uint4*>(base)[k ^ pk];
  } else {
    const int hb = (bl >> 2) & 1;  // 8-byte half swap within a piece (slot bit 2)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint2* p = reinterpret_cast<const uint2*>(base) + 2 * (k ^ pk);
      const uint2 lo = p[hb], hi = p[hb ^ 1];
      raw[k] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
}

// The value of the lane whose block index differs in bit M (M = 1, 2 within
// a quad, M = 4 within an eight-lane group), one 32-bit half through DPP.
template <int M>
__device__ __forceinline__ int dpp_pair(int v) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else {
    // Lanes 0-3 of each eight read lanes 4-7 (row_shl:4, banks 0 and 2),
    // lanes 4-7 read lanes 0-3 (row_shr:4, banks 1 and 3).
    const int o = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);
    return __builtin_amdgcn_update_dpp(o, v, 0x114, 0xF, 0xA, false);
  }
}

// Hadamard stage over block bit M (lane partner bl ^ M) paired with register
// bit Q.  The pair (lower lane, upper lane) holds, at each slot i with bit Q
// clear, a = lower's value and c = upper's value of the same channel offset
// (the upper lane's slots are relabeled, so slot i | Q of each lane holds
// what its partner needs): one exchange of slot i | Q gives each lane the
// other's value, and each lane then keeps both outputs a + c (slot i) and
// a - c (slot i | Q) for its half of the offsets.  Afterwards block bit M
// stands for channel bit log2 Q and register bit Q for the block bit; the
// upper lane's a - c comes out negated.
template <int M, int Q>
__device__ __forceinline__ void lane_stage(double (&x)[32]) {
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if (r & Q) {
      const int lo = dpp_pair<M>(__double2loint(x[r]));
      const int hi = dpp_pair<M>(__double2hiint(x[r]));
      const double recv = __hiloint2double(hi, lo), own = x[r ^ Q];
      x[r ^ Q] = own + recv;
      x[r] = own - recv;
    }
  }
}

// Rotation of the tile in `raw` into the LDS tile, then the factor vectors
// reset.  The LDS tile holds sigma_j (X H_D)_tj: the rotation without its
// 1/sqrt(D) and with a sign sigma_j = chan_negated(j) ? -1 : 1 per channel,
// both undone where they matter (see seal_finish; the Sinkhorn factors c_j
// do not depend on a common scale of the tile or on the signs).  The sums
// run in float64, where they are exact (a sum of at most 256 fp16 values
// needs at most 48 significant bits), and are rounded to fp32 once: in fp32,
// channels whose rotated value nearly cancels would keep rounding noise of
// the size of the value itself.
//
// Butterflies over the five in-register bits run first; over a relabeled
// slot bit the upper lane's pair is stored swapped, which a lane sign s
// absorbs (new low = s a + b, new high = a - s b).  Then one lane_stage per
// block bit.  Channel of slot r in lane bl afterwards (D 128):
// r[0..2] | bl1 << 3 | bl0 << 4 | r4 << 5 | r3 << 6; at D 256 slot bits 0, 1,
// bl2, bl1, bl0, r4, r3, r2.  Ends with a barrier.
template <int D>
__device__ __forceinline__ void seal_rotate(const uint4 (&raw)[4], SealSmem<D>& sm, int tid) {
  constexpr int NB = D / 32;
  const int tl = tid / NB, bl = tid % NB;
  double x[32];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t ws[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * k + 2 * e] = (double)h2f((uint16_t)(ws[e] & 0xFFFFu));
      x[8 * k + 2 * e + 1] = (double)h2f((uint16_t)(ws[e] >> 16));
    }
  }
  const int rl = rot_relabel<D>(bl);
#pragma unroll
  for (int st = 1; st < 32; st <<= 1) {
    const double s = (rl & st) ? -1.0 : 1.0;
    const bool relabeled = st == 16 || st == 8 || (NB == 8 && st == 4);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & st)) {
        const double a = x[i], b = x[i + st];
        if (relabeled) {
          x[i] = fma(s, a, b);
          x[i + st] = fma(-s, b, a);
        } else {
          x[i] = a + b;
          x[i + st] = a - b;
        }
      }
    }
  }
  lane_stage<1, 16>(x);
  lane_stage<2, 8>(x);
  if constexpr (NB == 8) lane_stage<4, 4>(x);
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r2 = p & 1, r3 = (p >> 1) & 1, r4 = p >> 2;
    const int g = NB == 4 ? (r2 | ((bl >> 1) << 1) | ((bl & 1) << 2) | (r4 << 3) | (r3 << 4))
                          : (((bl >> 2) & 1) | (((bl >> 1) & 1) << 1) | ((bl & 1) << 2) | (r4 << 3) | (r3 << 4) |
                             (r2 << 5));
    *reinterpret_cast<float4*>(xg(sm, tl, g)) =
        make_float4((float)x[4 * p], (float)x[4 * p + 1], (float)x[4 * p + 2], (float)x[4 * p + 3]);
  }
  if (tid < D) {
    sm.u[sk(tid)] = 1.0f / D;
    sm.c2[tid] = 1.0f;
  }
  lds_barrier();
}

// Sign that seal_rotate leaves on channel j of the LDS tile: each lane stage
// negates the channels whose block bit and paired channel bit are both set
// (channel bits 4 and 5, 3 and 6, and at D 256 2 and 7).
template <int D>
__device__ __forceinline__ bool chan_negated(int j) {
  const int m = (j >> 4) & (j >> 5) & 1;
  const int n = (j >> 3) & (j >> 6) & 1;
  const int o = D == 256 ? (j >> 2) & (j >> 7) & 1 : 0;
  return (m ^ n ^ o) != 0;
}

// Lane roles after the rotation.  Row role: tokens 2tp, 2tp+1 and channels
// 16cb .. 16cb+15, the RL = D/16 lanes of a token pair adjacent.  Column
// role: channels 2cp, 2cp+1 and tokens 16tb .. 16tb+15, the eight lanes of a
// channel pair adjacent.
template <int D>
struct SealRoles {
  static constexpr int RL = D / 16;
  static constexpr int RPW = 64 / RL;
  int tp, cb, cp, tb;
  __device__ explicit SealRoles(int tid) {
    const int w = tid >> 6, lane = tid & 63;
    tp = RPW * w + lane / RL;
    cb = lane % RL;
    cp = 8 * w + (lane >> 3);
    tb = lane & 7;
  }
};

// Sinkhorn iterations on the tile that seal_rotate left in LDS: A = X_r^2 in
// both roles' register blocks, then `iters` token and channel steps.  Leaves
// c_j^2 in sm.c2; ends with a barrier.
//
// Scaling: sm.u holds u_j = 1 / (D c_j^2), so the token step's plain sum
// sum_j A_tj u_j is r_t^2 itself, and the column role holds (D / T) A, so the
// channel step's sum sum_t (D / T) A_tj v_t is D c_j^2, whose reciprocal is
// the next u_j (powers of two only: exact).
//
// The lanes of a token pair (channel pair) with odd cb (tb) hold the pair in
// swapped order, so one DPP add gives every lane the sum of its own first
// token over itself and its neighbour: that folds both tokens into one value
// per lane, and the remaining steps of the reduction (same parity throughout)
// take one add each.  Lanes cb (tb) = 0 and 1 then hold the totals of the
// pair's first and second token (channel) and publish them together.
//
// Publishing: a new factor is 1 / total, kept finite with a min so that an
// all-zero row or column (total 0) has a factor that multiplies only zeros in
// the next step; its A entries are all zero, so the other steps do not change
// (the same as keeping its factor).  c_j^2 itself is stored in the last
// iteration only, 1 for an all-zero column (its factor stays 1).
template <int D>
__device__ __forceinline__ void seal_iterate(int iters, SealSmem<D>& sm, int tid) {
  constexpr int RL = SealRoles<D>::RL;
  const SealRoles<D> ro(tid);
  const int tp = ro.tp, cb = ro.cb, cp = ro.cp, tb = ro.tb;
  const int rsw = cb & 1, csw = tb & 1;
  float ar[2][16], ac[16][2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(xg(sm, 2 * tp + (r ^ rsw), 4 * cb + k));
      ar[r][4 * k] = a.x * a.x;
      ar[r][4 * k + 1] = a.y * a.y;
      ar[r][4 * k + 2] = a.z * a.z;
      ar[r][4 * k + 3] = a.w * a.w;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float* a = xg(sm, 16 * tb + i, cp >> 1) + 2 * (cp & 1);
    const float x0 = a[csw], x1 = a[csw ^ 1];
    ac[i][0] = x0 * x0 * (float)(D / kGroup);
    ac[i][1] = x1 * x1 * (float)(D / kGroup);
  }
  constexpr float kBig = 3.40282347e38f;

  for (int it = 0; it < iters; ++it) {
    // Token step: r_t^2 = mean_j A_tj u_j.
    {
      float uv[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(sm.u + 20 * cb + 4 * k);
        uv[4 * k] = q.x;
        uv[4 * k + 1] = q.y;
        uv[4 * k + 2] = q.z;
        uv[4 * k + 3] = q.w;
      }
      float pa = 0.f, pb = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        pa = fmaf(ar[0][c], uv[c], pa);
        pb = fmaf(ar[1][c], uv[c], pb);
      }
      float tot = pa + dpp_f<0xB1>(pb);  // quad_perm [1,0,3,2]
      tot += dpp_f<0x4E>(tot);           // quad_perm [2,3,0,1]
      tot += dpp_f<0x104>(tot);          // row_shl:4 (lanes 0, 1 of each eight read 4, 5)
      if constexpr (RL == 16) tot += dpp_f<0x108>(tot);  // row_shl:8
      asm volatile("" : "+v"(tot));  // the last add stays outside the branch, merged with its DPP move
      if (cb < 2) sm.v[sk(2 * tp + cb)] = fminf(__builtin_amdgcn_rcpf(tot), kBig);
    }
    lds_barrier();
    // Channel step: c_j^2 = mean_t A_tj v_t.
    {
      float vt[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(sm.v + 20 * tb + 4 * k);
        vt[4 * k] = q.x;
        vt[4 * k + 1] = q.y;
        vt[4 * k + 2] = q.z;
        vt[4 * k + 3] = q.w;
      }
      float qa = 0.f, qb = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        qa = fmaf(ac[i][0], vt[i], qa);
        qb = fmaf(ac[i][1], vt[i], qb);
      }
      float tot = qa + dpp_f<0xB1>(qb);
      tot += dpp_f<0x4E>(tot);
      tot += dpp_f<0x104>(tot);
      asm volatile("" : "+v"(tot));
      if (tb < 2) {
        sm.u[sk(2 * cp + tb)] = fminf(__builtin_amdgcn_rcpf(tot), kBig);
        if (it == iters - 1) sm.c2[2 * cp + tb] = tot > 0.f ? tot * (1.0f / D) : 1.f;
      }
    }
    lds_barrier();
  }
}

// Code of a value y = x / step + mid that lies in [0, 2^BITS - 1] up to a few
// fp32 rounding errors (|x| / step <= (2^BITS - 1) / 2 by the choice of the
// step): adding 2^23 rounds y to an integer, half to even, as rintf does, and
// leaves that integer in the low mantissa bits; a y a little below 0 (above
// 2^BITS - 1) rounds to 0 (2^BITS - 1), so no clamp is needed.
// The bit pattern is 0x4B000000 + code; pack16 removes the constant part.
constexpr uint32_t kRtnMagicBits = 0x4B000000u;
template <int BITS>
__device__ __forceinline__ uint32_t rtn_code(float y) {
  return __float_as_uint(y + 8388608.0f);
}

// Sixteen codes of one record row as a little-endian bit stream: code e
// occupies bits [BITS e, BITS e + BITS) of the words (the whole-row layout
// restricted to one 16-code block, which starts on a byte boundary).  The
// inputs are rtn_code patterns, kRtnMagicBits + code: the words are built
// with adds (the code fields do not overlap, so an add is an or for them),
// and the shifted copies of the constant, the same for every call, are
// subtracted at the end.
template <int BITS>
struct PackBias {
  uint32_t w[(16 * BITS + 31) / 32];
  constexpr PackBias() : w{} {
    for (int e = 0; e < 16; ++e) {
      const int bit = BITS * e;
      w[bit / 32] += kRtnMagicBits << (bit % 32);
      if (bit % 32 + BITS > 32) w[bit / 32 + 1] += kRtnMagicBits >> (32 - bit % 32);
    }
  }
};

template <int BITS>
__device__ __forceinline__ void pack16(const uint32_t (&code)[16], uint32_t (&w)[(16 * BITS + 31) / 32]) {
  constexpr PackBias<BITS> bias;
  constexpr int NW = (16 * BITS + 31) / 32;
#pragma unroll
  for (int k = 0; k < NW; ++k) w[k] = 0u - bias.w[k];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int bit = BITS * e;
    w[bit / 32] += code[e] << (bit % 32);
    if (bit % 32 + BITS > 32) w[bit / 32 + 1] += code[e] >> (32 - bit % 32);
  }
}

// Store the 2*BITS bytes of a packed 16-code block at dst (dst is 2*BITS
// bytes into a row: 4-byte aligned when BITS is even, 2-byte aligned else).
template <int BITS>
__device__ __forceinline__ void store16(uint8_t* dst, const uint32_t (&w)[(16 * BITS + 31) / 32]) {
  if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int k = 0; k < BITS / 2; ++k) reinterpret_cast<uint32_t*>(dst)[k] = w[k];
  } else {
#pragma unroll
    for (int k = 0; k < BITS; ++k)
      reinterpret_cast<uint16_t*>(dst)[k] = (uint16_t)((k & 1) ? (w[k / 2] >> 16) : (w[k / 2] & 0xFFFFu));
  }
}

// Channel and token scales, round to nearest and packing of the tile that
// seal_iterate left (X_r in LDS, c_j^2 in sm.c2) into record `rec`.  Every
// global store comes last, after all of the phase's arithmetic: a store's
// source registers may not be reused before it completes, and waiting for a
// store also waits for every global load issued before it (one in-order
// counter), which would expose the next tile's prefetch.
// 1/sqrt(D), the rotation's normalization (float).
template <int D>
constexpr float kRotScale = D == 128 ? 0.0883883476483184405f : 0.0625f;

template <int D, int BITS, bool TOKEN_MAJOR>
__device__ __forceinline__ void seal_finish(uint8_t* __restrict__ rec, float* __restrict__ dbg, SealSmem<D>& sm,
                                            int tid) {
  constexpr int LEVELS = (1 << BITS) - 1;
  constexpr float MID = 0.5f * LEVELS;
  constexpr int CODE_BYTES = kGroup * D * BITS / 8;
  constexpr int RL = SealRoles<D>::RL;
  constexpr int NW = (16 * BITS + 31) / 32;  // 32-bit words holding 16 codes
  const SealRoles<D> ro(tid);
  const int tp = ro.tp, cb = ro.cb, cp = ro.cp, tb = ro.tb;

  // ---- channel scales ----------------------------------------------------
  // cinv carries sigma_j, so X_r / c_j below is (sigma_j X H_D)_tj * cinv_j
  // up to the common factor sqrt(D), which cancels in the codes and is
  // applied to the token scales.
  float cj = 0.f;
  if (tid < D) {
    cj = sqrtf(sm.c2[tid]);
    sm.cinv[sk(tid)] = (chan_negated<D>(tid) ? -1.0f : 1.0f) / cj;
  }
  lds_barrier();

  // ---- token scales from the largest |X_r / c| of each token (row role) ---
  float zr[2][16];
  float inv[2], sc[2];
  {
    float ci[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 q = *reinterpret_cast<const float4*>(sm.cinv + 20 * cb + 4 * k);
      ci[4 * k] = q.x;
      ci[4 * k + 1] = q.y;
      ci[4 * k + 2] = q.z;
      ci[4 * k + 3] = q.w;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = *reinterpret_cast<const float4*>(xg(sm, 2 * tp + r, 4 * cb + k));
        zr[r][4 * k] = a.x * ci[4 * k];
        zr[r][4 * k + 1] = a.y * ci[4 * k + 1];
        zr[r][4 * k + 2] = a.z * ci[4 * k + 2];
        zr[r][4 * k + 3] = a.w * ci[4 * k + 3];
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) mx = fmaxf(mx, fabsf(zr[r][c]));
      mx = max_rl<RL>(mx);
      inv[r] = mx > 0.f ? (float)LEVELS / (2.0f * mx) : 0.f;
      sc[r] = mx * (2.0f / LEVELS * kRotScale<D>);
    }
    if (cb == 0) *reinterpret_cast<float2*>(sm.inv + sk(2 * tp)) = make_float2(inv[0], inv[1]);
  }

  // ---- codes -------------------------------------------------------------
  // K record: tokens 2tp, 2tp+1, channels [16 cb, 16 cb + 16) (row role).
  // V record: channels 2cp, 2cp+1, tokens [16 tb, 16 tb + 16) (column role).
  uint32_t out[2][NW];
  if constexpr (TOKEN_MAJOR) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint32_t code[16];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        code[e] = rtn_code<BITS>(fmaf(zr[r][e], inv[r], MID));
      pack16<BITS>(code, out[r]);
    }
  } else {
    lds_barrier();
    const float2 ci = *reinterpret_cast<const float2*>(sm.cinv + sk(2 * cp));
    float zc[16][2], iv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float2 a = *reinterpret_cast<const float2*>(xg(sm, 16 * tb + i, cp >> 1) + 2 * (cp & 1));
      zc[i][0] = a.x * ci.x;
      zc[i][1] = a.y * ci.y;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 q = *reinterpret_cast<const float4*>(sm.inv + 20 * tb + 4 * k);
      iv[4 * k] = q.x;
      iv[4 * k + 1] = q.y;
      iv[4 * k + 2] = q.z;
      iv[4 * k + 3] = q.w;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t code[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        code[i] = rtn_code<BITS>(fmaf(zc[i][c], iv[i], MID));
      pack16<BITS>(code, out[c]);
    }
  }

  // ---- stores ------------------------------------------------------------
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    uint8_t* dst = TOKEN_MAJOR ? rec + (size_t)(2 * tp + r) * (D * BITS / 8) + cb * (16 * BITS / 8)
                               : rec + (size_t)(2 * cp + r) * (kGroup * BITS / 8) + tb * (16 * BITS / 8);
    store16<BITS>(dst, out[r]);
  }
  if (cb == 0) {
    const uint32_t s2 = (uint32_t)f2h_rne(sc[0]) | ((uint32_t)f2h_rne(sc[1]) << 16);
    *reinterpret_cast<uint32_t*>(rec + CODE_BYTES + 4 * tp) = s2;
    if (dbg) *reinterpret_cast<float2*>(dbg + 2 * tp) = make_float2(sc[0], sc[1]);
  }
  if (tid < D) {
    reinterpret_cast<uint16_t*>(rec + CODE_BYTES + 2 * kGroup)[tid] = f2h_rne(cj);
    if (dbg) dbg[kGroup + tid] = cj;
  }
}

// seal_finish for a width known only at run time (uniform over the
// workgroup): one branch per width, so a kernel serves every (K, V) width
// pair without an instance per pair.
template <int D, bool TOKEN_MAJOR>
__device__ __forceinline__ void seal_finish_bits(int bits, uint8_t* __restrict__ rec, SealSmem<D>& sm, int tid) {
  switch (bits) {
    case 2: seal_finish<D, 2, TOKEN_MAJOR>(rec, nullptr, sm, tid); break;
    case 3: seal_finish<D, 3, TOKEN_MAJOR>(rec, nullptr, sm, tid); break;
    case 4: seal_finish<D, 4, TOKEN_MAJOR>(rec, nullptr, sm, tid); break;
    case 5: seal_finish<D, 5, TOKEN_MAJOR>(rec, nullptr, sm, tid); break;
    case 6: seal_finish<D, 6, TOKEN_MAJOR>(rec, nullptr, sm, tid); break;
    default: seal_finish<D, 8, TOKEN_MAJOR>(rec, nullptr, sm, tid); break;
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------
template <int D, int BITS, int KIND>
__global__ __launch_bounds__(kSealThreadsPerD * D) void seal_tiles_kernel(const __half* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int64_t dst_stride, float* __restrict__ dbg, int iters) {
  __shared__ SealSmem<D> sm;
  const int64_t i = blockIdx.x;
  uint4 raw[4];
  load_tile<D>(raw, src + i * kGroup * D, threadIdx.x);
  seal_rotate<D>(raw, sm, threadIdx.x);
  seal_iterate<D>(iters, sm, threadIdx.x);
  seal_finish<D, BITS, KIND == 0>(dst + i * dst_stride, dbg ? dbg + i * (kGroup + D) : nullptr, sm, threadIdx.x);
}

// Tile idx of a bulk seal (group g, request-head bh, K|V, layer; tile index
// g + G (bh + NBH (kind + 2 layer))): its fp16 source and record, or false
// if the request has no such group or the group has no storage.  len(b) is
// request b's prompt length.
template <int D, typename Len>
__device__ __forceinline__ bool prefill_tile(const SealPrefillArgs& a, int idx, Len len, const __half*& src,
                                             uint8_t*& rec, int& kind) {
  const int g = idx % a.gmax, r = idx / a.gmax;
  const int bhl = r % a.nbh, r2 = r / a.nbh;
  const int layer = r2 >> 1;
  kind = r2 & 1;
  if (kSink + kGroup * (g + 1) > len(bhl / a.hkv)) return false;
  const PrefillLayer& L = a.layer[layer];
  const int64_t bh = (int64_t)a.b0 * a.hkv + bhl;
  const int64_t off = pair_offset(L.map, (int)(bh / a.hkv), (int)(bh % a.hkv), g, a.hkv, a.max_groups, a.group_bytes);
  if (off < 0) return false;
  src = (kind ? L.v : L.k) + (bh * a.src_tokens + kSink + (int64_t)kGroup * g) * D;
  rec = L.records + off + (kind ? a.rec_k_bytes : 0);
  return true;
}

// Bulk sealing at D 128: one workgroup per tile, two resident per CU.
// One tile per workgroup lets the dispatcher refill a CU as soon as either of
// its two workgroups finishes.  (A persistent grid that prefetched its next
// tile during the iterations measured slower: the older workgroup of a CU
// takes issue priority and finishes its share early, leaving the younger
// one alone on the CU for the last tiles.)
template <int D>
__global__ __launch_bounds__(kSealThreadsPerD * D) void seal_prefill_kernel(SealPrefillArgs a) {
  __shared__ SealSmem<D> sm;
  const int idx = blockIdx.x;
  const int tslot = idx * (kSealThreadsPerD * D / 64) + (int)(threadIdx.x >> 6);  // trace build only
  trace_begin(tslot);
  const __half* src;
  uint8_t* rec;
  int kind;
  if (!prefill_tile<D>(a, idx, [&](int b) { return a.lens.len[b]; }, src, rec, kind)) return;
  uint4 raw[4];
  load_tile<D>(raw, src, threadIdx.x);
  seal_rotate<D>(raw, sm, threadIdx.x);
  trace_mark(tslot, 1);  // tile loaded and rotated
  seal_iterate<D>(a.iters, sm, threadIdx.x);
  trace_mark(tslot, 2);  // iterations done
  if (kind == 0)
    seal_finish_bits<D, true>(a.k_bits, rec, sm, threadIdx.x);
  else
    seal_finish_bits<D, false>(a.v_bits, rec, sm, threadIdx.x);
  trace_mark(tslot, 3);  // record stores issued
}

// Bulk sealing at D 256, where one workgroup (136 KB of LDS) fills a CU: a
// resident grid whose workgroups take tiles blockIdx.x, + gridDim.x, ... and
// load the next tile into registers before finishing the current one, so
// the load does not leave the CU idle at each tile's start.
template <int D>
__global__ __launch_bounds__(kSealThreadsPerD * D) void seal_prefill_persistent_kernel(SealPrefillArgs a) {
  __shared__ SealSmem<D> sm;
  __shared__ int32_t s_len[kMaxPrefillBatch];   // prompt lengths: LDS reads in the loop wait for nothing else
  constexpr int kWavesPerTile = kSealThreadsPerD * D / 64;
  int tid = threadIdx.x;
  for (int b = tid; b < kMaxPrefillBatch; b += kSealThreadsPerD * D) s_len[b] = a.lens.len[b];
  __syncthreads();
  auto len = [&](int b) { return s_len[b]; };
  int idx = blockIdx.x;
  const __half* src;
  uint8_t* rec;
  int kind;
  while (idx < a.n_tiles && !prefill_tile<D>(a, idx, len, src, rec, kind)) idx += gridDim.x;
  if (idx >= a.n_tiles) return;
  uint4 raw[4];
  load_tile<D>(raw, src, tid);
  for (;;) {
    // The per-lane index math of the phases is recomputed per tile rather
    // than kept live across the loop (it would not fit the registers).
    asm volatile("" : "+v"(tid));
    const int tslot = idx * kWavesPerTile + (tid >> 6);  // trace build only
    trace_begin(tslot);
    seal_rotate<D>(raw, sm, tid);
    trace_mark(tslot, 1);  // tile loaded and rotated
    int nidx = idx + (int)gridDim.x;
    const __half* nsrc = nullptr;
    uint8_t* nrec = nullptr;
    int nkind = 0;
    while (nidx < a.n_tiles && !prefill_tile<D>(a, nidx, len, nsrc, nrec, nkind)) nidx += gridDim.x;
    if (nidx < a.n_tiles) load_tile<D>(raw, nsrc, tid);   // lands during the iterations
    seal_iterate<D>(a.iters, sm, tid);
    trace_mark(tslot, 2);  // iterations done
    if (kind == 0)
      seal_finish_bits<D, true>(a.k_bits, rec, sm, tid);
    else
      seal_finish_bits<D, false>(a.v_bits, rec, sm, tid);
    trace_mark(tslot, 3);  // record stores issued
    if (nidx >= a.n_tiles) break;
    idx = nidx;
    rec = nrec;
    kind = nkind;
    lds_barrier();   // every wave is done with this tile's LDS before the next rotation writes it
  }
}

// Seal on arrival.  Workgroup (entry, KV head, K|V): in the predicate form
// the entry is request x / hkv; in the list form it is list entry x / hkv,
// naming request req[i] and group group[i].  Either way the group sealed is
// the one whose 128 tokens fill the request's tail, g = (n - 128) / 128 - 1
// with n = seq_len[b] >= 256 and (n - 128) % 128 == 0; a list entry naming
// another group, or a request outside [0, batch), is skipped.
template <int D>
__global__ __launch_bounds__(kSealThreadsPerD * D) void seal_stream_kernel(SealStreamArgs a) {
  __shared__ SealSmem<D> sm;
  const int e = blockIdx.x / a.hkv, h = blockIdx.x - (blockIdx.x / a.hkv) * a.hkv;
  const int kind = blockIdx.y;
  const int b = a.req ? a.req[e] : e;
  if (b < 0 || b >= a.batch) return;
  const int n = a.seq_len[b];
  if (n < kSink + kGroup || ((n - kSink) % kGroup) != 0) return;
  const int g = (n - kSink) / kGroup - 1;
  if (g >= a.max_groups || (a.req && a.group[e] != g)) return;
  const int64_t off = pair_offset(a.map, b, h, g, a.hkv, a.max_groups, a.group_bytes);
  if (off < 0) return;
  const __half* src = (kind ? a.tail_v : a.tail_k) + ((int64_t)b * a.hkv + h) * kGroup * D;
  uint8_t* rec = a.records + off + (kind ? a.rec_k_bytes : 0);
  uint4 raw[4];
  load_tile<D>(raw, src, threadIdx.x);
  seal_rotate<D>(raw, sm, threadIdx.x);
  seal_iterate<D>(a.iters, sm, threadIdx.x);
  if (kind == 0)
    seal_finish_bits<D, true>(a.k_bits, rec, sm, threadIdx.x);
  else
    seal_finish_bits<D, false>(a.v_bits, rec, sm, threadIdx.x);
}

// Append one token and seal the group it completes, in one launch: workgroup
// (request-head bh, K|V) writes its row of the new token, and if that row
// completes the tail it seals the tail into the group's record.  Every
// workgroup needs the request's old length n, so the length can only advance
// once all 2 Hkv workgroups of the request have read it: each adds
// 1 << kArriveShift to seq_len[b] (a device-scope atomic that also returns
// n in the low bits), and the one that finds the count complete removes the
// count and adds the token.
template <int D>
__global__ __launch_bounds__(kSealThreadsPerD * D) void append_seal_kernel(AppendSealArgs a) {
  __shared__ SealSmem<D> sm;
  __shared__ int s_n;
  const int bh = blockIdx.x, kind = blockIdx.y;
  const int b = bh / a.hkv;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const uint32_t nwg = 2u * (uint32_t)a.hkv;
    uint32_t* len = reinterpret_cast<uint32_t*>(a.seq_len + b);
    const uint32_t old = atomicAdd(len, 1u << kArriveShift);
    const int n = (int)(old & kLenMask);
    if ((old >> kArriveShift) == nwg - 1) atomicAdd(len, (n < a.cap ? 1u : 0u) - (nwg << kArriveShift));
    s_n = n;
  }
  __syncthreads();
  const int n = s_n;
  if (n >= a.cap) return;
  const int slot = n < kSink ? n : (n - kSink) % kGroup;
  __half* row = (n < kSink ? (kind ? a.sink_v : a.sink_k) : (kind ? a.tail_v : a.tail_k)) +
                ((int64_t)bh * kGroup + slot) * D;
  if (tid < D / 8)
    reinterpret_cast<uint4*>(row)[tid] = reinterpret_cast<const uint4*>((kind ? a.v_new : a.k_new) + (int64_t)bh * D)[tid];
  const int n1 = n + 1;
  if (n1 < kSink + kGroup || (n1 - kSink) % kGroup != 0) return;
  const int g = (n1 - kSink) / kGroup - 1;
  if (g >= a.max_groups) return;
  const int64_t off = pair_offset(a.map, b, bh - b * a.hkv, g, a.hkv, a.max_groups, a.group_bytes);
  if (off < 0) return;
  __syncthreads();  // the row written above is part of the tile read below
  const __half* tile = (kind ? a.tail_v : a.tail_k) + (int64_t)bh * kGroup * D;
  uint8_t* rec = a.records + off + (kind ? a.rec_k_bytes : 0);
  uint4 raw[4];
  load_tile<D>(raw, tile, tid);
  seal_rotate<D>(raw, sm, tid);
  seal_iterate<D>(a.iters, sm, tid);
  if (kind == 0)
    seal_finish_bits<D, true>(a.k_bits, rec, sm, tid);
  else
    seal_finish_bits<D, false>(a.v_bits, rec, sm, tid);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int BITS>
static hipError_t launch_tiles_db(int kind, const void* src, void* dst, int64_t stride, float* dbg, int n, int iters,
                                  hipStream_t st) {
  if (kind == 0)
    hipLaunchKernelGGL((seal_tiles_kernel<D, BITS, 0>), dim3(n), dim3(kSealThreadsPerD * D), 0, st, (const __half*)src,
                       (uint8_t*)dst, stride, dbg, iters);
  else
    hipLaunchKernelGGL((seal_tiles_kernel<D, BITS, 1>), dim3(n), dim3(kSealThreadsPerD * D), 0, st, (const __half*)src,
                       (uint8_t*)dst, stride, dbg, iters);
  return hipGetLastError();
}

hipError_t launch_seal_tiles(int D, int bits, int kind, const void* src, void* dst, int64_t stride, float* dbg, int n,
                             int iters, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
#define CALL(d, b) e = launch_tiles_db<d, b>(kind, src, dst, stride, dbg, n, iters, st)
  KVARN_DISPATCH_DB(D, bits, CALL);
#undef CALL
  return e;
}

template <int D>
static void launch_prefill_t(const SealPrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((seal_prefill_kernel<D>), dim3(a.n_tiles), dim3(kSealThreadsPerD * D), 0, st, a);
}

// Resident workgroups of the persistent D 256 seal on the current device
// (0 if the query fails), looked up once per device.
static int persistent_seal_wgs() {
  static std::atomic<int> cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  int v = dev < 16 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (v > 0) return v;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, seal_prefill_persistent_kernel<256>,
                                                   kSealThreadsPerD * 256, 0) != hipSuccess)
    return 0;
  v = per_cu * decode_cu_count();
  if (dev < 16 && v > 0) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_seal_prefill(int D, const SealPrefillArgs& args, int max_groups_in_batch, int nbh, hipStream_t st) {
  if (max_groups_in_batch <= 0 || nbh <= 0) return hipSuccess;
  SealPrefillArgs a = args;
  a.gmax = max_groups_in_batch;
  a.nbh = nbh;
  a.n_tiles = 2 * a.n_layers * nbh * max_groups_in_batch;
  if (D == 128) {
    launch_prefill_t<128>(a, st);
  } else {
    const int wgs = persistent_seal_wgs();
    if (wgs > 0)
      hipLaunchKernelGGL((seal_prefill_persistent_kernel<256>), dim3(std::min(wgs, a.n_tiles)),
                         dim3(kSealThreadsPerD * 256), 0, st, a);
    else
      launch_prefill_t<256>(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_append_seal(int D, const AppendSealArgs& a, int nbh, hipStream_t st) {
  if (nbh <= 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL((append_seal_kernel<128>), dim3(nbh, 2), dim3(kSealThreadsPerD * 128), 0, st, a);
  else
    hipLaunchKernelGGL((append_seal_kernel<256>), dim3(nbh, 2), dim3(kSealThreadsPerD * 256), 0, st, a);
  return hipGetLastError();
}

#ifdef KVARN_WAVE_TRACE
hipError_t trace_io_seal(void* host, size_t bytes) { return trace_io_local(host, bytes); }
#endif

hipError_t launch_seal_stream(int D, const SealStreamArgs& a, int nbh, hipStream_t st) {
  if (nbh <= 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL((seal_stream_kernel<128>), dim3(nbh, 2), dim3(kSealThreadsPerD * 128), 0, st, a);
  else
    hipLaunchKernelGGL((seal_stream_kernel<256>), dim3(nbh, 2), dim3(kSealThreadsPerD * 256), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvarn
