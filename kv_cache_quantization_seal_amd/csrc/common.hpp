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

}  // namespace kvarn
