// Device helpers shared by the KVarN HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

constexpr int kGroup = 128;  // tokens per sealed group
constexpr int kSink = 128;   // exact leading tokens
constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}
__device__ __forceinline__ uint16_t f2h_rne(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// Order LDS traffic between lanes of one wave (no cross-wave barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reductions across the 16 lanes of one DPP row (lanes 16r .. 16r+15), every
// lane receiving the result: swap neighbours, swap pairs, mirror within the
// half row, mirror within the row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}
// Maximum over the whole wave of an unsigned value (or of a non-negative
// float's bit pattern, which orders like the value): DPP within each row,
// then the four row results through scalar registers.  All lanes active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u) {
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, true));
  const uint32_t r0 = __builtin_amdgcn_readlane(u, 0), r1 = __builtin_amdgcn_readlane(u, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(u, 32), r3 = __builtin_amdgcn_readlane(u, 48);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ float wave_max_nonneg(float v) {
  return __uint_as_float(wave_max_u32(__float_as_uint(v)));
}
// Sum of v over lanes l and l^16 (resp. l^32), in every lane, through the
// gfx950 row/half swaps (no LDS traffic).
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Whole-wave maximum / sum of a float (DPP rows, then the four row results
// through scalar registers as bit patterns); every lane receives the result.
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Position p (0..15) of an unpacked 16-code block -> code index within the
// block, for the unpacking used by the decode kernel:
//   2-bit: dword w -> bytes (w >> 2k) & 0x03030303, k = 0..3: byte b of
//          dword k is code 4b + k;
//   4-bit: dwords w0,w1 -> w0 & M, (w0 >> 4) & M, w1 & M, (w1 >> 4) & M with
//          M = 0x0F0F0F0F: byte b of dword k is code 8(k/2) + 2b + (k%2).
//   other widths: byte p is code p (natural order).
template <int BITS>
__host__ __device__ constexpr int unpack_index(int p) {
  return BITS == 2 ? 4 * (p & 3) + (p >> 2)
                   : BITS == 4 ? 8 * ((p >> 2) >> 1) + 2 * (p & 3) + ((p >> 2) & 1) : p;
}

// Unpack one 16-code block (BITS*2 bytes) into 16 int8 MFMA operand bytes
// (widths 2 and 4).
template <int BITS>
__device__ __forceinline__ v4i unpack16(const uint32_t* w) {
  v4i r;
  if constexpr (BITS == 2) {
    const uint32_t x = w[0];
    r[0] = (int)(x & 0x03030303u);
    r[1] = (int)((x >> 2) & 0x03030303u);
    r[2] = (int)((x >> 4) & 0x03030303u);
    r[3] = (int)((x >> 6) & 0x03030303u);
  } else {
    r[0] = (int)(w[0] & 0x0F0F0F0Fu);
    r[1] = (int)((w[0] >> 4) & 0x0F0F0F0Fu);
    r[2] = (int)(w[1] & 0x0F0F0F0Fu);
    r[3] = (int)((w[1] >> 4) & 0x0F0F0F0Fu);
  }
  return r;
}

// Block s (16 codes) of a lane's chunk of N dwords of one record row, as 16
// int8 MFMA operand bytes in unpack_index order.  Widths 2 and 4 keep their
// mask-and-shift order; 8-bit codes are offset by -128 to fit int8 (the
// caller corrects the mid level for that); 3, 5 and 6 bits are extracted in
// natural order from the row's little-endian bit stream.
template <int BITS, int N>
__device__ __forceinline__ v4i unpack_block(const uint32_t (&c)[N], int s) {
  if constexpr (BITS == 2) {
    return unpack16<2>(&c[s]);
  } else if constexpr (BITS == 4) {
    return unpack16<4>(&c[2 * s]);
  } else if constexpr (BITS == 8) {
    v4i r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = (int)(c[4 * s + k] ^ 0x80808080u);
    return r;
  } else {
    v4i r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t d = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bit = 16 * BITS * s + BITS * (4 * k + e);
        const int wi = bit / 32, sh = bit % 32;
        uint32_t v;
        if (sh + BITS <= 32)
          v = (c[wi] >> sh) & ((1u << BITS) - 1);
        else
          v = __builtin_amdgcn_alignbit(c[wi + 1], c[wi], sh) & ((1u << BITS) - 1);
        d |= v << (8 * e);
      }
      r[k] = (int)d;
    }
    return r;
  }
}

// Magic-number rounding: for |x| < 2^22, x + 1.5*2^23 rounds x to the nearest
// integer (ties to even) in the low mantissa bits, whose low byte is then
// rint(x) as a two's complement int8.
constexpr float kMagic = 12582912.0f;

// Three radix-128 int8 limbs of the real number y*inv (|y*inv| <= 127.5):
// y*inv ~ a0 + a1/128 + a2/128^2, |error| <= 0.5/128^2.  Returns the three
// magic-rounded floats; limb i is the low byte of f[i].
__device__ __forceinline__ void limbs_r128(float y, float inv, float& f0, float& f1, float& f2) {
  f0 = fmaf(y, inv, kMagic);
  const float a0 = f0 - kMagic;
  const float t1 = fmaf(y, inv, -a0);
  f1 = fmaf(t1, 128.0f, kMagic);
  const float a1 = f1 - kMagic;
  const float t2 = fmaf(t1, 128.0f, -a1);
  f2 = fmaf(t2, 128.0f, kMagic);
}

// Low bytes of four magic-rounded floats -> one dword (byte 0 = first).
__device__ __forceinline__ uint32_t pack_low_bytes(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Split x (|x| <= 127.5) into three int8 limbs a0 + a1/254 + a2/254^2 with
// round-to-nearest at each level; returns the limbs as exact floats.
__device__ __forceinline__ void limbs3(float x, float& a0, float& a1, float& a2) {
  a0 = rintf(x);
  float r1 = (x - a0) * 254.0f;
  a1 = rintf(r1);
  float r2 = (r1 - a1) * 254.0f;
  a2 = rintf(r2);
}

// Pack four exact small integers (as floats, in [-128, 127]) into one dword of
// int8 bytes (byte 0 = first).
__device__ __forceinline__ uint32_t pack4_i8(float a, float b, float c, float d) {
  const uint32_t x0 = (uint32_t)((int)a) & 0xFFu;
  const uint32_t x1 = (uint32_t)((int)b) & 0xFFu;
  const uint32_t x2 = (uint32_t)((int)c) & 0xFFu;
  const uint32_t x3 = (uint32_t)((int)d) & 0xFFu;
  return x0 | (x1 << 8) | (x2 << 16) | (x3 << 24);
}


// Workgroup barrier that orders LDS accesses only: global loads and stores
// issued before it stay in flight (a full __syncthreads also makes this
// wave's global stores visible, which on this target waits for every
// outstanding global access, loads included).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Position of 16-byte group g (channels 4g .. 4g+3) within row t of an fp32
// [128][P] LDS tile, P = 4 (mod 32) dwords.  LDS serves a 128-bit access
// eight lanes at a time from 32 four-byte banks, so eight lanes are
// conflict-free when their groups land on eight different bank quads.  With
// the low three bits of g XORed by ((g >> 3) ^ (t >> 4)) & 7 that holds for
// eight lanes reading 4-channel group k of sixteen-channel blocks 0..7 of one
// row, for eight lanes reading one group of rows t, t+16, ..., t+112, and for
// eight lanes of consecutive rows (the row pitch moves them one quad each).
__device__ __forceinline__ int xgrp(int g, int t) { return g ^ (((g >> 3) ^ (t >> 4)) & 7); }

// Natural-order Sylvester Hadamard transform (unnormalized) of token rows held
// as 64-channel slices: thread (t, rb) holds channels [64 rb, 64 rb + 64) of
// token t in x.  The butterflies over the six low channel-index bits run in
// registers; for D > 64 the block-index bits are combined through LDS
// (xs = [128][P] fp32 scratch, which this overwrites; with SWZ its 16-byte
// groups sit at xgrp positions).  Contains barriers: all threads of the block
// must call it.
template <int D, int P, bool SWZ = false>
__device__ __forceinline__ void rotate_row_slice(float (&x)[64], float* xs, int t, int rb) {
  constexpr int NB = D / 64;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (!(i & s)) {
        const float a = x[i], b = x[i + s];
        x[i] = a + b;
        x[i + s] = a - b;
      }
    }
  }
  if constexpr (NB > 1) {
    auto grp = [&](int g) { return xs + t * P + 4 * (SWZ ? xgrp(g, t) : g); };
#pragma unroll
    for (int k = 0; k < 16; ++k)
      *reinterpret_cast<float4*>(grp(16 * rb + k)) = make_float4(x[4 * k], x[4 * k + 1], x[4 * k + 2], x[4 * k + 3]);
    __syncthreads();
    // y_{64 rb + i} = sum_o (-1)^popcount(rb & o) x_{64 o + i}
    const float own = (__popc(rb) & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] *= own;
#pragma unroll
    for (int o = 0; o < NB; ++o) {
      if (o == rb) continue;
      const float sg = (__popc(rb & o) & 1) ? -1.0f : 1.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(grp(16 * o + k));
        x[4 * k] = fmaf(sg, q.x, x[4 * k]);
        x[4 * k + 1] = fmaf(sg, q.y, x[4 * k + 1]);
        x[4 * k + 2] = fmaf(sg, q.z, x[4 * k + 2]);
        x[4 * k + 3] = fmaf(sg, q.w, x[4 * k + 3]);
      }
    }
    __syncthreads();
  }
}

}  // namespace kvarn
