// KVarN decode attention on gfx950 (the kernel templates): split-K over
// sealed groups, exact sink and tail, one inverse rotation per query head.
// The split kernel is instantiated in one translation unit per K code width
// (decode_k<b>.hip), so the instances compile in parallel; plan, combine and
// dispatch are in decode.hip.
//
// The query is rotated by the same Hadamard matrix as the stored K and V, so
// q.k is unchanged and attention over the records runs in the rotated frame;
// the record part of the output is rotated back once per query head
// ["KVarN KV Cache: Implementation and Benchmarks" (anbeeld.com), §1 "Where
// KVarN Comes From"].  Sink and tail are exact fp16 and are read in the
// original frame; records are read directly, never expanded in memory (same
// page, §2.1 "Sink, Body, And Tail").
//
// Record splits.  A record workgroup is four independent waves; each wave
// takes an even share of the sealed groups of one (request, KV head) and
// processes each group alone, its operands loaded from HBM straight into
// registers in MFMA operand order (the next group's loads are issued while
// the current one is computed):
//   logit_t = s^K_t * sum_j q~_j (code_tj - mid),  q~ = q_r * c^K * scale,
//   w_t = p_t * s^V_t,  o_rot_j += c^V_j * sum_t w_t (code_tj - mid).
// Both sums run on v_mfma_i32_16x16x64_i8 with the codes as exact int8
// operands.  q~ and w are split into three radix-128 int8 limbs
// x * inv ~ a0 + a1/128 + a2/128^2 (|error| <= 0.5/128^2 of the group maximum
// scaled to the top-limb range); the 16 MFMA rows carry (head, limb) pairs,
// so each lane holds every limb of one head and recombines them exactly in
// int32, with one conversion to fp32.  Softmax is base-2 online softmax per
// wave; the four waves merge through LDS once, at the end of the split.
//
// Operand layouts (lane l, lane group G = l/16, n = l%16):
//   * B operand of QK = K codes: column n of N-tile nt is token tok(nt, n);
//     lane group G holds channel blocks cb = G*KS + s (16 channels each,
//     KS = D/64 K-steps); the unpacked byte p of block cb is channel
//     16 cb + unpack_index<KB>(p).
//   * A operand of QK = q~ limbs from LDS, row m = 4h + limb, same K slots.
//   * A operand of PV = w limbs from LDS, row m = 4h + limb; lane group G,
//     step s holds token block tb = 2G + s, byte p = token 16 tb +
//     unpack_index<VB>(p).
//   * B operand of PV = V codes (channel-major rows): column n of N-tile ct
//     is channel 16 ct + n, same token slots.
//   tok(nt, n) = 16 (n/2) + unpack_index<VB>(8 (n%2) + nt): the w limbs of
//   lane n sit at LDS bytes 8n + nt.
#pragma once

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace kvarn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kExactTok = 16;     // exact tokens per wave per round
// The exact tokens of a pair (sink 128 + tail < 128) go to 4 exact splits of
// one round (64 tokens each) or to 2 exact splits of two rounds (128 each);
// the plan chooses (plan_decode).

typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int D, int KB, int VB>
struct RecGeom {
  static constexpr int KS = D / 64;                      // QK K-steps
  static constexpr int NCT = D / 16;                     // PV channel tiles
  static constexpr int NTT = kGroup / 16;                // QK token tiles
  static constexpr int LBK = KS * 2 * KB;                // K-code bytes per lane per token
  static constexpr int LBV = 4 * VB;                     // V-code bytes per lane per channel
  static constexpr int KROW = D * KB / 8;                // bytes of one token row of K codes
  static constexpr int VROW = kGroup * VB / 8;           // bytes of one channel row of V codes
  static constexpr int KCODE = kGroup * D * KB / 8;
  static constexpr int VCODE = kGroup * D * VB / 8;
  static constexpr int KREC = KCODE + 2 * kGroup + 2 * D;
  static constexpr int VREC = VCODE + 2 * kGroup + 2 * D;
  static constexpr int GB = KREC + VREC;                 // bytes per group (K record | V record)
  static constexpr int QB = D / 16;                      // q~ operand bytes per producer lane
};

template <int D, int GQ>
struct alignas(16) WaveLds {
  alignas(16) uint8_t ql[GQ][3][D];       // q~ limbs, QK A-operand order
  alignas(16) uint8_t wl[GQ][3][kGroup];  // w limbs, PV A-operand order
};

template <int D, int KB, int VB, int GQ>
struct alignas(16) RecSmem {
  WaveLds<D, GQ> wv[kWaves];
  float mm[kWaves][GQ];         // per-wave partial maxima
  float ll[kWaves][GQ];         // per-wave partial sums
  float oo[kWaves][GQ][D];      // per-wave partial outputs (rotated frame)
};

template <int D, int GQ>
struct alignas(16) ExactSmem {
  alignas(16) uint16_t v[kWaves][kExactTok][D + 8];  // V rows of one round (fp16)
  alignas(16) float p[kWaves][kExactTok][4];         // softmax numerators [token][head]
  float qx[GQ][D];
  float mm[kWaves][GQ];
  float ll[kWaves][GQ];
  float oo[kWaves][GQ][D];
};

// N dwords from global memory (16-byte pieces where N allows).
template <int N>
__device__ __forceinline__ void load_dw_global(uint32_t (&dst)[N], const void* src) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const uint4 x = reinterpret_cast<const uint4*>(src)[i];
      dst[4 * i] = x.x;
      dst[4 * i + 1] = x.y;
      dst[4 * i + 2] = x.z;
      dst[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = reinterpret_cast<const uint32_t*>(src)[i];
  }
}

// Rotated, scaled query of one head as the q~ producer lanes need it, by the
// wave alone (no LDS, no barrier).  Lane j (0..15) of the head's 16-lane row
// holds channels QB j .. QB j + QB - 1 in `w` (fp16 pairs).  The Hadamard
// butterflies run over the low channel bits in registers and over the lane
// bits across the row (DPP: quad_perm for 1 and 2, masked row shifts for 4,
// row_ror for 8; the upper lane of a pair keeps lower - upper).  Operand
// byte i of lane j is channel 16 (j/2) + unpack_index<KB>(8 (j%2) + i) (QB 8)
// or 16 j + unpack_index<KB>(i) (QB 16); for 2-bit K codes at QB 8 half of
// those channels sit in lane j^1.  The result is q H_D / sqrt(D) times
// scale * log2(e) (zero for an invalid head).
template <int D, int QB, int KB>
__device__ __forceinline__ void rotate_query(const uint32_t (&w)[QB / 2], bool valid, int j, float scale,
                                             float (&qr)[QB]) {
  float x[QB];
#pragma unroll
  for (int i = 0; i < QB / 2; ++i) {
    x[2 * i] = valid ? h2f((uint16_t)(w[i] & 0xFFFFu)) : 0.f;
    x[2 * i + 1] = valid ? h2f((uint16_t)(w[i] >> 16)) : 0.f;
  }
#pragma unroll
  for (int st = 1; st < QB; st <<= 1) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      if (!(i & st)) {
        const float u = x[i], v = x[i + st];
        x[i] = u + v;
        x[i + st] = u - v;
      }
    }
  }
#pragma unroll
  for (int st = 1; st < 16; st <<= 1) {
    const bool hi = j & st;
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const int v = __float_as_int(x[i]);
      int o;
      if (st == 1) {
        o = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
      } else if (st == 2) {
        o = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
      } else if (st == 4) {
        o = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0, 2
        o = __builtin_amdgcn_update_dpp(o, v, 0x114, 0xF, 0xA, false);  // row_shr:4, banks 1, 3
      } else {
        o = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true);   // row_ror:8
      }
      const float pv = __int_as_float(o);
      x[i] = hi ? pv - x[i] : x[i] + pv;
    }
  }
  const float f = scale * kLog2e * ((D == 128) ? 0.08838834764831845f : 0.0625f);
#pragma unroll
  for (int i = 0; i < QB; ++i) x[i] *= f;
  if constexpr (QB == 8 && KB == 2) {
    // Channel offset m within the 16-channel block: lane 2(j/2) holds
    // m = 0..7, lane 2(j/2)+1 holds m = 8..15.
    float nb[QB];
#pragma unroll
    for (int i = 0; i < QB; ++i) nb[i] = dpp_f<0xB1>(x[i]);
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const int m0 = 4 * (i & 3) + (i >> 2);      // j even
      const int m1 = 4 * (i & 3) + 2 + (i >> 2);  // j odd
      const float ve = m0 < 8 ? x[m0 & 7] : nb[m0 & 7];
      const float vo = m1 < 8 ? nb[m1 & 7] : x[m1 & 7];
      qr[i] = (j & 1) ? vo : ve;
    }
  } else {
#pragma unroll
    for (int i = 0; i < QB; ++i) qr[i] = x[QB == 8 ? (KB == 4 ? 2 * (i & 3) + (i >> 2) : i) : unpack_index<KB>(i)];
  }
}

template <int VB>
__device__ __forceinline__ int tok_of(int nt, int n) {
  return 16 * (n >> 1) + unpack_index<VB>(8 * (n & 1) + nt);
}

// Buffer resource over `bytes` bytes at a wave-uniform base; loads past the
// end return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Largest |top limb| 2^m - 1 so that sum_j A_j (2 code_j - L) fits int32,
// with A_j = a0*2^14 + a1*2^7 + a2 and |a1|,|a2| <= 64, over k_terms terms:
// k L (a0max 2^14 + 8256) < 2^31.
__host__ __device__ constexpr float top_limb(int k_terms, int levels) {
  int t = 127;
  while (t > 1 && (double)k_terms * levels * ((double)t * 16384.0 + 8256.0) >= 2147483648.0) t >>= 1;
  return (float)t;
}

__device__ __forceinline__ void store_partial_ml(const DecodeArgs& a, int b, int hq_idx, int split, float m, float l) {
  const int64_t row = ((int64_t)b * a.hq + hq_idx) * a.nsplit + split;
  a.ws_ml[2 * row] = m;
  a.ws_ml[2 * row + 1] = l;
}

// ---------------------------------------------------------------------------
// Record split: four independent waves, each streaming whole groups.
// ---------------------------------------------------------------------------

// One group's operands as one lane holds them, loaded straight from the
// record in MFMA operand order (loop-invariant per-lane offsets):
//   k[nt]  K codes of token tok(nt, n), channel blocks of lane group G;
//   v[ct]  V codes of channel NCT*n + ct, token blocks 2G, 2G+1;
//   sk/sv  s^K, s^V of the lane's eight tokens tok(0..7, n): half 2(nt&3) +
//          (nt>>2) of the four dwords;
//   ck     c^K of the q~ producer's channels; cv  c^V of channels NCT*n + ct.
template <int D, int KB, int VB>
struct Stage {
  using Gm = RecGeom<D, KB, VB>;
  uint32_t k[Gm::NTT][Gm::LBK / 4];
  uint32_t v[Gm::NCT][Gm::LBV / 4];
  uint32_t sk[4], sv[4];
  uint32_t ck[Gm::QB / 2];
  uint32_t cv[Gm::NCT / 2];
  bool live;  // the K part came from a stored group (else it reads as zeros)
};

// N dwords at byte offset `off` of a buffer: 16-byte loads when N is a
// multiple of 4 (those offsets are 16-byte aligned), else 8- or 4-byte ones.
template <int N>
__device__ __forceinline__ void load_dw(uint32_t (&dst)[N], __amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (N % 4 != 0 && N > 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0);
  } else if constexpr (N == 1) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (N == 2) {
    const v2u x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    dst[0] = x.x;
    dst[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
      dst[4 * i] = x.x;
      dst[4 * i + 1] = x.y;
      dst[4 * i + 2] = x.z;
      dst[4 * i + 3] = x.w;
    }
  }
}

__device__ __forceinline__ float half_of(const uint32_t* w, int i) {
  return h2f((uint16_t)((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu)));
}

template <int D, int KB, int VB, int GQ, bool PAGED>
__device__ void record_split(RecSmem<D, KB, VB, GQ>& sm, const DecodeArgs& a, int b, int kvh, int split,
                             int nseq) {
  using Gm = RecGeom<D, KB, VB>;
  using St = Stage<D, KB, VB>;
  constexpr int KS = Gm::KS, NCT = Gm::NCT, NTT = Gm::NTT, QB = Gm::QB;
  constexpr int LK = (1 << KB) - 1, LV = (1 << VB) - 1;
  constexpr float QMAX = top_limb(D, LK);
  constexpr float WMAX = top_limb(kGroup, LV);
  // 8-bit codes enter the MFMAs offset by -128: sum q (2 code - L) =
  // 2 sum q (code - 128) - (L - 256) sum q.
  constexpr int LKE = KB == 8 ? LK - 256 : LK, LVE = VB == 8 ? LV - 256 : LV;
  // Token order of a lane's eight tokens (see tok_of) and the half index of
  // token nt in the lane's s^K / s^V dwords.
  auto tstep = [](int nt) { return VB == 2 ? 4 * (nt & 3) + (nt >> 2) : VB == 4 ? 2 * (nt & 3) + (nt >> 2) : nt; };
  auto shalf = [](int nt) { return (VB == 2 || VB == 4) ? 2 * (nt & 3) + (nt >> 2) : nt; };
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int G = l >> 4, n = l & 15;
  const bool hvalid = G < GQ;         // QK/PV output row of this lane is head G
  const int hm = n >> 2, im = n & 3;  // A-operand row of this lane: (head, limb)
  const bool arow_valid = hm < GQ && im < 3;
  WaveLds<D, GQ>& wv = sm.wv[w];
  const int tslot = (int)blockIdx.x * kWaves + w;  // trace build only

  // The pair's sealed groups (from its current length, not the capacity the
  // grid was planned for) are shared evenly over its record waves: wave
  // wi = 4 split + w takes groups [G wi / nw, G (wi+1) / nw), nw = 4 n_rec_splits,
  // i.e. floor or ceil of G / nw consecutive groups (at most groups_per_wave).
  const int n_groups = nseq > kSink ? min((nseq - kSink) / kGroup, a.c.max_groups) : 0;
  const int nw = a.n_rec_splits * kWaves, wi = split * kWaves + w;
  const int ga = (int)((int64_t)n_groups * wi / nw);
  const int gb = (int)((int64_t)n_groups * (wi + 1) / nw);

  // Per-lane byte offsets within a group (loop-invariant).
  // Tokens tok(0..7, n) are tok0 + tstep(nt): tok0 = 16(n/2) + 2(n&1) and
  // steps 4(nt&3) + (nt>>2) (2-bit V), tok0 = 8n and steps 2(nt&3) + (nt>>2)
  // (4-bit V) or nt (other widths): a lane base plus a constant.
  const int tok0 = VB == 2 ? 16 * (n >> 1) + 2 * (n & 1) : 8 * n;
  const int kbase = tok0 * Gm::KROW + G * Gm::LBK;
  auto kofs = [&](int nt) { return kbase + tstep(nt) * Gm::KROW; };
  const int skofs = Gm::KCODE + 2 * tok0;
  const int svofs = Gm::KREC + Gm::VCODE + 2 * tok0;
  // q~ producer lane: head hq = l/16, operand bytes [QB*j, QB*j + QB), j = l%16.
  const int hq = l >> 4, j = l & 15;
  int ckofs;
  if constexpr (QB == 8)
    ckofs = Gm::KCODE + 2 * kGroup + 2 * (16 * (j >> 1) + (KB == 2 ? 2 * (j & 1) : 8 * (j & 1)));
  else
    ckofs = Gm::KCODE + 2 * kGroup + 2 * (16 * j);
  const int cvofs = Gm::KREC + Gm::VCODE + 2 * kGroup + 2 * NCT * n;
  const int vbase = Gm::KREC + NCT * n * Gm::VROW + G * Gm::LBV;
  auto vofs = [&](int ct) { return vbase + ct * Gm::VROW; };

  // Byte offset of group g's record pair, or -1 for a group past the wave's
  // range or with no storage.  Wave-uniform: a paged cache's block table is
  // read with a scalar load (its own counter, so waiting for it never waits
  // for the record loads in flight).
  const int64_t pair_base = (((int64_t)b * a.c.hkv + kvh) * a.c.max_groups) * a.c.group_bytes;
  auto group_off = [&](int g, bool on) -> int64_t {
    if (!on) return -1;
    if constexpr (!PAGED) return pair_base + (int64_t)g * a.c.group_bytes;
    typedef const __attribute__((address_space(4))) int32_t ConstI32;
    const int blk = *(ConstI32*)(a.c.map.table + (int64_t)b * a.c.max_groups + g);
    return (blk >= 0 && blk < a.c.map.num_blocks) ? ((int64_t)blk * a.c.hkv + kvh) * a.c.group_bytes : -1;
  };
  // Wave-uniform buffer range of a group; an unused range is empty, so its
  // loads return zero without touching memory and every path issues the
  // same loads.
  auto rsrc_at = [&](int64_t off) {
    const uint64_t addr = reinterpret_cast<uint64_t>(a.c.records + (off >= 0 ? off : 0));
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const int bytes = __builtin_amdgcn_readfirstlane(off >= 0 ? Gm::GB : 0);
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), bytes);
  };
  // K part (c^K first: it is needed first), V part (s^V first).
  auto load_k = [&](St& S, int64_t off) {
    S.live = off >= 0;
    const __amdgpu_buffer_rsrc_t r = rsrc_at(off);
    if constexpr (QB == 8 && KB == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) S.ck[k] = __builtin_amdgcn_raw_buffer_load_b32(r, ckofs + 8 * k, 0, 0);
    } else {
      load_dw(S.ck, r, ckofs);
    }
    if constexpr (VB != 2) {
      load_dw(S.sk, r, skofs);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) S.sk[k] = __builtin_amdgcn_raw_buffer_load_b32(r, skofs + 8 * k, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) load_dw(S.k[nt], r, kofs(nt));
  };
  auto load_v = [&](St& S, int64_t off) {
    const __amdgpu_buffer_rsrc_t r = rsrc_at(off);
    if constexpr (VB != 2) {
      load_dw(S.sv, r, svofs);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) S.sv[k] = __builtin_amdgcn_raw_buffer_load_b32(r, svofs + 8 * k, 0, 0);
    }
    load_dw(S.cv, r, cvofs);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) load_dw(S.v[ct], r, vofs(ct));
  };

  // The query's loads go out first: loads complete in issue order, so waiting
  // for the query must not also wait for the group loads behind it.
  const bool qvalid = hq < GQ;
  uint32_t qw[QB / 2];
  load_dw_global<QB / 2>(qw, a.q + (((int64_t)b * a.hq + kvh * GQ + (qvalid ? hq : 0)) * D + QB * j));
  __builtin_amdgcn_sched_barrier(0);
  St SA;
  const int64_t off0 = group_off(ga, ga < gb);
  load_k(SA, off0);
  load_v(SA, off0);
  __builtin_amdgcn_sched_barrier(0);

  // q~ producer values (scaled query in the log2 domain, rotated), per wave.
  float qr[QB];
  rotate_query<D, QB, KB>(qw, qvalid, j, a.scale, qr);
  trace_mark(tslot, 1);  // query loaded and rotated
  auto ckh = [](int i) {
    return QB == 8 ? ((KB == 2 || KB == 4) ? 2 * (i & 3) + (i >> 2) : i) : unpack_index<KB>(i);
  };

  float m_run = -INFINITY, l_run = 0.f;  // head G
  float o_acc[NCT];                      // head G, channel NCT*n + ct
#pragma unroll
  for (int c = 0; c < NCT; ++c) o_acc[c] = 0.f;

  // One group from stage S; each half of the stage is refilled with group gn
  // as soon as it has been consumed (K part after QK, V part after PV), so
  // the next group's loads overlap most of this group's work.
  auto process = [&](St& S, int gn) {
    const int64_t offn = group_off(gn, gn < gb);  // issued early: used after QK
    const bool live = !PAGED || S.live;  // this group is stored (a paged table may leave it out)
    // q~ limbs of head hq with E = max |q~| over the head's channels (one
    // DPP row per head).
    float y[QB];
    float ym = 0.f;
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      y[i] = qr[i] * half_of(S.ck, ckh(i));
      ym = fmaxf(ym, fabsf(y[i]));
    }
    const float E = row16_max(ym);  // row G == head G: also the QK scale of this lane
    if (gn == ga + 1) trace_mark(tslot, 2);  // first group's c^K arrived
    {
      const float inv = E > 0.f ? QMAX * __builtin_amdgcn_rcpf(E) : 0.f;
      uint32_t b0[QB / 4], b1[QB / 4], b2[QB / 4];
#pragma unroll
      for (int i = 0; i < QB / 4; ++i) {
        float f0[4], f1[4], f2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) limbs_r128(y[4 * i + e], inv, f0[e], f1[e], f2[e]);
        b0[i] = pack_low_bytes(f0[0], f0[1], f0[2], f0[3]);
        b1[i] = pack_low_bytes(f1[0], f1[1], f1[2], f1[3]);
        b2[i] = pack_low_bytes(f2[0], f2[1], f2[2], f2[3]);
      }
      if (qvalid) {
        uint8_t* base = &wv.ql[hq][0][QB * j];
        if constexpr (QB == 8) {
          *reinterpret_cast<v2u*>(base) = v2u{b0[0], b0[1]};
          *reinterpret_cast<v2u*>(base + D) = v2u{b1[0], b1[1]};
          *reinterpret_cast<v2u*>(base + 2 * D) = v2u{b2[0], b2[1]};
        } else {
          *reinterpret_cast<v4u*>(base) = v4u{b0[0], b0[1], b0[2], b0[3]};
          *reinterpret_cast<v4u*>(base + D) = v4u{b1[0], b1[1], b1[2], b1[3]};
          *reinterpret_cast<v4u*>(base + 2 * D) = v4u{b2[0], b2[1], b2[2], b2[3]};
        }
      }
    }
    wave_sync();

    // QK over the eight token tiles.
    v4i aq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (arow_valid) {
        const uint4 v = *reinterpret_cast<const uint4*>(&wv.ql[hm][im][16 * (G * KS + s)]);
        aq[s] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {
        aq[s] = v4i{0, 0, 0, 0};
      }
    }
    v4i sacc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[s], ones, sacc, 0, 0, 0);
    const uint32_t negls =
        0u - (uint32_t)LKE * (((uint32_t)sacc[0] << 14) + ((uint32_t)sacc[1] << 7) + (uint32_t)sacc[2]);
    const float kscale = E * (1.0f / (QMAX * 32768.0f));
    float logit[NTT];
    float lmax = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[s], unpack_block<KB>(S.k[nt], s), acc, 0, 0, 0);
      const uint32_t x = ((uint32_t)acc[0] << 14) + ((uint32_t)acc[1] << 7) + (uint32_t)acc[2];
      const int yv = (int)((x << 1) + negls);
      logit[nt] = (hvalid && live) ? (float)yv * (half_of(S.sk, shalf(nt)) * kscale) : -INFINITY;
      lmax = fmaxf(lmax, logit[nt]);
    }
    if (gn == ga + 1) trace_mark(tslot, 3);  // first group's QK done
    load_k(S, offn);

    // Softmax update; w = p * s^V with its exact per-head maximum W.
    const float gmax = row16_max(lmax);
    const float m_new = fmaxf(m_run, gmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float wv_[NTT];
    float psum = 0.f, wm = 0.f;
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) {
      const float p = (hvalid && live) ? __builtin_amdgcn_exp2f(logit[nt] - m_new) : 0.f;
      psum += p;
      wv_[nt] = p * half_of(S.sv, shalf(nt));
      wm = fmaxf(wm, wv_[nt]);
    }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int c = 0; c < NCT; ++c) o_acc[c] *= alpha;
    const float W = row16_max(wm);
    {
      const float winv = W > 0.f ? WMAX * __builtin_amdgcn_rcpf(W) : 0.f;
      uint32_t b0[2], b1[2], b2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float f0[4], f1[4], f2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) limbs_r128(wv_[4 * hh + e], winv, f0[e], f1[e], f2[e]);
        b0[hh] = pack_low_bytes(f0[0], f0[1], f0[2], f0[3]);
        b1[hh] = pack_low_bytes(f1[0], f1[1], f1[2], f1[3]);
        b2[hh] = pack_low_bytes(f2[0], f2[1], f2[2], f2[3]);
      }
      if (hvalid) {
        // Token tok(nt, n) sits at PV operand byte 8n + nt.
        uint8_t* base = &wv.wl[G][0][8 * n];
        *reinterpret_cast<v2u*>(base) = v2u{b0[0], b0[1]};
        *reinterpret_cast<v2u*>(base + kGroup) = v2u{b1[0], b1[1]};
        *reinterpret_cast<v2u*>(base + 2 * kGroup) = v2u{b2[0], b2[1]};
      }
    }
    wave_sync();

    // PV over the channel tiles.
    v4i aw[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (arow_valid) {
        const uint4 v = *reinterpret_cast<const uint4*>(&wv.wl[hm][im][16 * (2 * G + s)]);
        aw[s] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {
        aw[s] = v4i{0, 0, 0, 0};
      }
    }
    v4i tacc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) tacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[s], ones, tacc, 0, 0, 0);
    const uint32_t neglt =
        0u - (uint32_t)LVE * (((uint32_t)tacc[0] << 14) + ((uint32_t)tacc[1] << 7) + (uint32_t)tacc[2]);
    const float vscale = W * (1.0f / (WMAX * 32768.0f));
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[s], unpack_block<VB>(S.v[ct], s), acc, 0, 0, 0);
      const uint32_t x = ((uint32_t)acc[0] << 14) + ((uint32_t)acc[1] << 7) + (uint32_t)acc[2];
      const int yv = (int)((x << 1) + neglt);
      o_acc[ct] = fmaf((float)yv * vscale, half_of(S.cv, ct), o_acc[ct]);
    }
    if (gn == ga + 1) trace_mark(tslot, 4);  // first group's PV done
    load_v(S, offn);
    wave_sync();  // this group's limbs have been read before the next group writes
  };

  for (int g = ga; g < gb; ++g) process(SA, g + 1);
  trace_mark(tslot, 5);  // every group done

  // Merge the four waves' partials (m replicated per head; l summed over the
  // row; o over disjoint channels) and write this split's partial.
  const float lw = row16_sum(l_run);
  if (hvalid) {
    if (n == 0) {
      sm.mm[w][G] = m_run;
      sm.ll[w][G] = lw;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) sm.oo[w][G][NCT * n + ct] = o_acc[ct];
  }
  __syncthreads();
  for (int idx = tid; idx < GQ * D; idx += 256) {
    const int h = idx / D, ch = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) M = fmaxf(M, sm.mm[k][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        const float mw = sm.mm[k][h];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L = fmaf(f, sm.ll[k][h], L);
        O = fmaf(f, sm.oo[k][h][ch], O);
      }
    }
    const int64_t row = ((int64_t)b * a.hq + kvh * GQ + h) * a.nsplit + split;
    a.ws_o[row * D + ch] = O;
    if (ch == 0) store_partial_ml(a, b, kvh * GQ + h, split, M, L);
  }
  trace_mark(tslot, 6);  // partial written
}

// ---------------------------------------------------------------------------
// Exact split: the sink and the tail, fp16, original frame.  Exact split es
// covers exact tokens [P es, P es + P), P = 64 kExactRounds (the sink's tokens
// first, then the tail's); wave w takes kExactRounds rounds of 16 of them;
// lane (token, quarter) holds a quarter of a K row and of a V row.  QK: fp32
// FMAs against the LDS query; PV: V rows staged in LDS.
// ---------------------------------------------------------------------------
// With the append folded into the step, whether request b's token may ride
// in the decode launches by its device length n: it completes no group and
// the cache is not full (the caller's host lengths promised this; a request
// for which they were wrong is left without its token instead of having it
// written to a wrong slot).
__device__ __forceinline__ bool fold_ok(const DecodeArgs& a, int n) {
  const int cap = kSink + kGroup * a.c.max_groups + kGroup - 1;
  const int n1 = n + 1;
  return a.k_new && n < cap && !(n1 >= kSink + kGroup && (n1 - kSink) % kGroup == 0);
}

template <int D, int GQ, int kExactRounds>
__device__ void exact_split(ExactSmem<D, GQ>& sm, const DecodeArgs& a, int b, int kvh, int es, int split, int n,
                            bool fold) {
  constexpr int kExactPerSplit = kWaves * kExactTok * kExactRounds;  // exact tokens of this split
  constexpr int QD = D / 4;     // channels per lane (quarter row)
  constexpr int CPLX = D / 64;  // channels per lane in the PV part
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int quarter = l >> 4, tl = l & 15;
  const int n_sink = min(n, kSink);
  const int tau = n > kSink ? (n - kSink) % kGroup : 0;
  const int n_exact = max(0, n_sink + tau);
  const int64_t bh = (int64_t)b * a.c.hkv + kvh;

  // Query loads first, then both rounds' K and V quarter rows (an invalid
  // token reads sink row 0, which always exists, and is masked later).
  constexpr int QPT = (GQ * D + 255) / 256;
  __half qh[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int idx = tid + 256 * i;
    qh[i] = idx < GQ * D ? a.q[((int64_t)b * a.hq + kvh * GQ) * D + idx] : __half(0.f);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 kr[kExactRounds][QD / 8], vr[kExactRounds][QD / 8];
  bool valid[kExactRounds], dst_tail[kExactRounds];
  int64_t dst[kExactRounds];  // element offset of the appended token's quarter row, or -1
#pragma unroll
  for (int round = 0; round < kExactRounds; ++round) {
    const int e = kExactPerSplit * es + kExactTok * (kExactRounds * w + round) + tl;
    valid[round] = e < n_exact;
    const bool in_tail = valid[round] && e >= n_sink;
    const int64_t row = bh * kGroup + (valid[round] ? (in_tail ? e - n_sink : e) : 0);
    // With the append folded in, the newest position (the last exact token)
    // comes from the step's input; its slot is written below.
    const bool fresh = fold && valid[round] && e == n_exact - 1;
    const __half* ks = fresh ? a.k_new + bh * D : (in_tail ? a.c.tail_k : a.c.sink_k) + row * D;
    const __half* vs = fresh ? a.v_new + bh * D : (in_tail ? a.c.tail_v : a.c.sink_v) + row * D;
    dst[round] = fresh ? row * D + quarter * QD : -1;
    dst_tail[round] = in_tail;
    const uint4* kp = reinterpret_cast<const uint4*>(ks + quarter * QD);
    const uint4* vp = reinterpret_cast<const uint4*>(vs + quarter * QD);
#pragma unroll
    for (int c = 0; c < QD / 8; ++c) {
      kr[round][c] = kp[c];
      vr[round][c] = vp[c];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < GQ * D) sm.qx[idx / D][idx % D] = __half2float(qh[i]) * a.scale * kLog2e;
  }
  __syncthreads();
  const int tslot = (int)blockIdx.x * kWaves + w;  // trace build only
  trace_mark(tslot, 1);  // query staged
  if (fold) {
#pragma unroll
    for (int round = 0; round < kExactRounds; ++round) {
      if (dst[round] >= 0) {
        uint4* kd = reinterpret_cast<uint4*>((dst_tail[round] ? a.c.tail_k : a.c.sink_k) + dst[round]);
        uint4* vd = reinterpret_cast<uint4*>((dst_tail[round] ? a.c.tail_v : a.c.sink_v) + dst[round]);
#pragma unroll
        for (int c = 0; c < QD / 8; ++c) {
          kd[c] = kr[round][c];
          vd[c] = vr[round][c];
        }
      }
    }
  }

  float m_run[GQ], l_run[GQ], o[GQ][CPLX];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CPLX; ++c) o[h][c] = 0.f;
  }
#pragma unroll
  for (int round = 0; round < kExactRounds; ++round) {
    const int e0 = kExactPerSplit * es + kExactTok * (kExactRounds * w + round);
    const bool ok = valid[round];
    float dot[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) dot[h] = 0.f;
    uint16_t* vrow = &sm.v[w][tl][quarter * QD];
#pragma unroll
    for (int c = 0; c < QD / 8; ++c)
      reinterpret_cast<uint4*>(vrow)[c] = ok ? vr[round][c] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < QD / 8; ++c) {
      const uint32_t ws[4] = {kr[round][c].x, kr[round][c].y, kr[round][c].z, kr[round][c].w};
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float4 qa = *reinterpret_cast<const float4*>(&sm.qx[h][quarter * QD + 8 * c]);
        const float4 qb = *reinterpret_cast<const float4*>(&sm.qx[h][quarter * QD + 8 * c + 4]);
        dot[h] = fmaf(qa.x, h2f((uint16_t)(ws[0] & 0xFFFFu)), dot[h]);
        dot[h] = fmaf(qa.y, h2f((uint16_t)(ws[0] >> 16)), dot[h]);
        dot[h] = fmaf(qa.z, h2f((uint16_t)(ws[1] & 0xFFFFu)), dot[h]);
        dot[h] = fmaf(qa.w, h2f((uint16_t)(ws[1] >> 16)), dot[h]);
        dot[h] = fmaf(qb.x, h2f((uint16_t)(ws[2] & 0xFFFFu)), dot[h]);
        dot[h] = fmaf(qb.y, h2f((uint16_t)(ws[2] >> 16)), dot[h]);
        dot[h] = fmaf(qb.z, h2f((uint16_t)(ws[3] & 0xFFFFu)), dot[h]);
        dot[h] = fmaf(qb.w, h2f((uint16_t)(ws[3] >> 16)), dot[h]);
      }
    }
    const bool valid_r = ok;
  float pt[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      // The four quarters of a row sum to the logit, after which every DPP
      // row holds the same 16 logits: row reductions give the round's
      // maximum and sum.
      float lg = xor32_sum(xor16_sum(dot[h]));
      lg = valid_r ? lg : -INFINITY;
      const float rmax = row16_max(lg);
      const float m_new = fmaxf(m_run[h], rmax);
      const float alpha = (m_run[h] == -INFINITY) ? 0.f : exp2f(m_run[h] - m_new);
      const float p = (valid_r && m_new != -INFINITY) ? exp2f(lg - m_new) : 0.f;
      pt[h] = p;
      l_run[h] = l_run[h] * alpha + row16_sum(p);
      m_run[h] = m_new;
#pragma unroll
      for (int c = 0; c < CPLX; ++c) o[h][c] *= alpha;
    }
    if (quarter == 0) {
#pragma unroll
      for (int h = 0; h < GQ; ++h) sm.p[w][tl][h] = pt[h];
    }
    wave_sync();
    const int nt = min(kExactTok, max(0, n_exact - e0));
    for (int t = 0; t < nt; ++t) {
      const float4 pv = *reinterpret_cast<const float4*>(&sm.p[w][t][0]);
      const float ph[4] = {pv.x, pv.y, pv.z, pv.w};
      float vf[CPLX];
      if constexpr (CPLX == 2) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(&sm.v[w][t][2 * l]);
        vf[0] = h2f((uint16_t)(x & 0xFFFFu));
        vf[1] = h2f((uint16_t)(x >> 16));
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(&sm.v[w][t][4 * l]);
        vf[0] = h2f((uint16_t)(x.x & 0xFFFFu));
        vf[1] = h2f((uint16_t)(x.x >> 16));
        vf[2] = h2f((uint16_t)(x.y & 0xFFFFu));
        vf[3] = h2f((uint16_t)(x.y >> 16));
      }
#pragma unroll
      for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int c = 0; c < CPLX; ++c) o[h][c] = fmaf(ph[h], vf[c], o[h][c]);
    }
    wave_sync();  // the staging rows are rewritten next round
  }
  trace_mark(tslot, 5);  // every round done
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    if (l == 0) {
      sm.mm[w][h] = m_run[h];
      sm.ll[w][h] = l_run[h];
    }
#pragma unroll
    for (int c = 0; c < CPLX; ++c) sm.oo[w][h][CPLX * l + c] = o[h][c];
  }
  __syncthreads();
  for (int idx = tid; idx < GQ * D; idx += 256) {
    const int h = idx / D, ch = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) M = fmaxf(M, sm.mm[k][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kWaves; ++k) {
        const float mw = sm.mm[k][h];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
        L = fmaf(f, sm.ll[k][h], L);
        O = fmaf(f, sm.oo[k][h][ch], O);
      }
    }
    const int64_t row = ((int64_t)b * a.hq + kvh * GQ + h) * a.nsplit + split;
    a.ws_o[row * D + ch] = O;
    if (ch == 0) store_partial_ml(a, b, kvh * GQ + h, split, M, L);
  }
  trace_mark(tslot, 6);  // partial written
}

template <int D, int KB, int VB, int GQ>
union DecodeSmemU {
  RecSmem<D, KB, VB, GQ> rec;
  ExactSmem<D, GQ> ex;
};

// 1-D grid of the record workgroups (pair-major) and the exact workgroups of
// every pair (n_exact_splits per pair), in the order the plan chose
// (record_first: record workgroups first).
template <int D, int KB, int VB, int GQ, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ DecodeSmemU<D, KB, VB, GQ> sm;
  trace_begin((int)blockIdx.x * kWaves + (int)(threadIdx.x >> 6));
  const int nex = a.nsplit - a.n_rec_splits;
  const int npair = a.c.batch * a.c.hkv;
  const int nrw = a.n_rec_splits * npair, nxw = nex * npair;
  const bool rec_first = a.record_first != 0;
  const int bx = blockIdx.x;
  if (rec_first ? bx >= nrw : bx < nxw) {
    const int ex = rec_first ? bx - nrw : bx;
    const int pair = ex / nex, es = ex - pair * nex;
    const int b = pair / a.c.hkv, kvh = pair - b * a.c.hkv;
    const int n = a.c.seq_len[b];
    const bool fold = fold_ok(a, n);   // the step's own token counts (append folded in)
    if (nex == 4)
      exact_split<D, GQ, 1>(sm.ex, a, b, kvh, es, a.n_rec_splits + es, n + fold, fold);
    else
      exact_split<D, GQ, 2>(sm.ex, a, b, kvh, es, a.n_rec_splits + es, n + fold, fold);
  } else {
    const int r = rec_first ? bx : bx - nxw;
    const int pair = r / a.n_rec_splits, split = r - pair * a.n_rec_splits;
    const int b = pair / a.c.hkv, kvh = pair - b * a.c.hkv;
    const int n = a.c.seq_len[b];
    record_split<D, KB, VB, GQ, PAGED>(sm.rec, a, b, kvh, split, n + fold_ok(a, n));
  }
}

// One workgroup (256 threads) per (query head, request): log-sum-exp merge of
// all splits, one inverse Hadamard of the record part, normalization.  The
// partial outputs do not depend on the weights, so every load is issued at
// once: lane l of every wave loads (max, sum) of splits l, l+64, ..., and wave
// w the partial outputs of splits w, w+4, ... for channels P*l .. P*l+P-1.
// Each wave then finds the maximum M and normalizer L itself, takes the
// weight of split s from lane s % 64, and one barrier joins the four sums.
// OPW: partial outputs per wave in the first batch (4 OPW splits; the host
// picks the smallest instance that covers the launch's splits, up to 80).
template <int D, int OPW>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int P = D / 64;
  static_assert(4 * OPW <= 2 * 64, "first-batch weights come from lanes of two (max, sum) passes");
  __shared__ float orec[kWaves][D];
  __shared__ float oex[kWaves][D];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int ns = a.nsplit, nrec = a.n_rec_splits;
  // Append folded into the step: the split kernel has attended over the new
  // token and stored it; the length moves on here, once per request (no
  // kernel of this launch reads it).  Read first, written last, so that the
  // read's round trip overlaps the loads of the partials instead of coming
  // before them.
  const bool advance = a.k_new && hq == 0 && tid == 0;
  const int n_old = advance ? a.c.seq_len[b] : 0;
  const int64_t base = ((int64_t)b * a.hq + hq) * ns;
  const float* ml = a.ws_ml + 2 * base;
  const float* ob = a.ws_o + base * D + P * l;
  auto load_o = [&](int s, float (&v)[P]) {
    const float* o = ob + (int64_t)s * D;
    if constexpr (P == 2) {
      const float2 x = *reinterpret_cast<const float2*>(o);
      v[0] = x.x;
      v[1] = x.y;
    } else {
      const float4 x = *reinterpret_cast<const float4*>(o);
      v[0] = x.x;
      v[1] = x.y;
      v[2] = x.z;
      v[3] = x.w;
    }
  };

  // (max, sum) of splits l and l + 64 in lane l (then further passes),
  // loaded first and unconditionally (clamped to the last split, masked
  // after): loads complete in issue order, so the weights can be formed
  // while the partial outputs behind them are still arriving.
  const float2 ml0 = *reinterpret_cast<const float2*>(ml + 2 * min(l, ns - 1));
  const float2 ml1 = *reinterpret_cast<const float2*>(ml + 2 * min(l + kWave, ns - 1));
  __builtin_amdgcn_sched_barrier(0);
  // First batch of this wave's partial outputs: splits w, w+4, ... (clamped
  // to the last split; the extra loads are discarded).
  float ov[OPW][P];
#pragma unroll
  for (int u = 0; u < OPW; ++u) load_o(min(w + kWaves * u, ns - 1), ov[u]);
  float m0 = l < ns ? ml0.x : -INFINITY, l0 = l < ns ? ml0.y : 0.f;
  float m1 = l + kWave < ns ? ml1.x : -INFINITY;
  float l1 = l + kWave < ns ? ml1.y : 0.f;
  float mloc = fmaxf(m0, m1);
  for (int s = l + 2 * kWave; s < ns; s += kWave) mloc = fmaxf(mloc, ml[2 * s]);
  const float M = wave_max_f(mloc);

  float ar[P], ae[P];
#pragma unroll
  for (int i = 0; i < P; ++i) ar[i] = ae[i] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    const float f0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
    const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    float lloc = fmaf(f0, l0, f1 * l1);
    for (int s = l + 2 * kWave; s < ns; s += kWave) {
      const float m = ml[2 * s];
      lloc += m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M) * ml[2 * s + 1];
    }
    L = wave_sum_f(lloc);
    auto add = [&](int s, float f, const float (&v)[P]) {
      if (s < nrec) {
#pragma unroll
        for (int i = 0; i < P; ++i) ar[i] = fmaf(f, v[i], ar[i]);
      } else {
#pragma unroll
        for (int i = 0; i < P; ++i) ae[i] = fmaf(f, v[i], ae[i]);
      }
    };
#pragma unroll
    for (int u = 0; u < OPW; ++u) {
      const int s = w + kWaves * u;
      if (s < ns) {
        // the weight of split s < 128 sits in lane s % 64 (f0 or f1)
        const float f = lane_f(s < kWave ? f0 : f1, s & (kWave - 1));
        add(s, f, ov[u]);
      }
    }
    // Splits past the first batch (long contexts): weight from its own max.
    for (int s = w + kWaves * OPW; s < ns; s += kWaves) {
      const float m = ml[2 * s];
      float v[P];
      load_o(s, v);
      add(s, m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M), v);
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    orec[w][P * l + i] = ar[i];
    oex[w][P * l + i] = ae[i];
  }
  __syncthreads();
  if (w != 0) return;
  float x[P], e[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    x[i] = (orec[0][P * l + i] + orec[1][P * l + i]) + (orec[2][P * l + i] + orec[3][P * l + i]);
    e[i] = (oex[0][P * l + i] + oex[1][P * l + i]) + (oex[2][P * l + i] + oex[3][P * l + i]);
  }
  // Inverse rotation of the record part (H symmetric): channel c = P*l + i;
  // butterflies over the bits of i in registers, over the bits of l across
  // lanes without LDS traffic: DPP for lane bits 1, 2, 4, 8 (the upper lane
  // of a pair keeps lower - upper), the row and half swaps for 16 and 32
  // (each lane gets the pair's sum s; the upper lane keeps s - 2 x).
#pragma unroll
  for (int st = 1; st < P; st <<= 1) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (!(i & st)) {
        const float u = x[i], v = x[i + st];
        x[i] = u + v;
        x[i + st] = u - v;
      }
    }
  }
#pragma unroll
  for (int st = 1; st < 16; st <<= 1) {
    const bool hi = l & st;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int v = __float_as_int(x[i]);
      int o;
      if (st == 1) {
        o = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
      } else if (st == 2) {
        o = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
      } else if (st == 4) {
        o = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0, 2
        o = __builtin_amdgcn_update_dpp(o, v, 0x114, 0xF, 0xA, false);  // row_shr:4, banks 1, 3
      } else {
        o = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true);   // row_ror:8
      }
      const float pv = __int_as_float(o);
      x[i] = hi ? pv - x[i] : x[i] + pv;
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const float s16 = xor16_sum(x[i]);
    x[i] = (l & 16) ? fmaf(-2.0f, x[i], s16) : s16;
    const float s32 = xor32_sum(x[i]);
    x[i] = (l & 32) ? fmaf(-2.0f, x[i], s32) : s32;
  }
  const float rs = (D == 128) ? 0.08838834764831845f : 0.0625f;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  float* out = a.out + ((int64_t)b * a.hq + hq) * D + P * l;
#pragma unroll
  for (int i = 0; i < P; ++i) out[i] = (x[i] * rs + e[i]) * inv;
  if (advance && fold_ok(a, n_old)) a.c.seq_len[b] = n_old + 1;
}

template <int D, int KB, int VB, int GQ>
static int resident_t(int dev) {
  // The smaller of the contiguous and the paged instances.
  int per_cu = 0, per_cu_paged = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<D, KB, VB, GQ, false>, 256, 0) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_paged, decode_split_kernel<D, KB, VB, GQ, true>, 256, 0) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return std::min(per_cu, per_cu_paged) * cus;
}

template <int D, int KB, int VB, int GQ>
static void launch_split_t(const DecodeArgs& a, hipStream_t st) {
  if (a.c.map.table)
    hipLaunchKernelGGL((decode_split_kernel<D, KB, VB, GQ, true>), dim3(a.nsplit * a.c.hkv * a.c.batch), dim3(256), 0,
                       st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, KB, VB, GQ, false>), dim3(a.nsplit * a.c.hkv * a.c.batch), dim3(256), 0,
                       st, a);
}

template <int D, int KB, int VB>
static void launch_split_g(int gq, const DecodeArgs& a, hipStream_t st) {
  if (gq == 1) launch_split_t<D, KB, VB, 1>(a, st);
  else if (gq == 2) launch_split_t<D, KB, VB, 2>(a, st);
  else launch_split_t<D, KB, VB, 4>(a, st);
}

template <int D, int KB, int VB>
static int resident_g(int gq, int dev) {
  return gq == 1 ? resident_t<D, KB, VB, 1>(dev) : gq == 2 ? resident_t<D, KB, VB, 2>(dev) : resident_t<D, KB, VB, 4>(dev);
}

// Every V width for the K width KB: the bodies of launch_split_k<KB> and
// resident_split_k<KB>, instantiated by decode_k<KB>.hip.
#define KVARN_FOR_VB(D, KB, VB, CALL)                                                    \
  do {                                                                                   \
    if (VB == 2) CALL(D, KB, 2); else if (VB == 3) CALL(D, KB, 3); else if (VB == 4) CALL(D, KB, 4); \
    else if (VB == 5) CALL(D, KB, 5); else if (VB == 6) CALL(D, KB, 6); else CALL(D, KB, 8);         \
  } while (0)

template <int KB>
static hipError_t launch_split_kb(int D, int vb, int gq, const DecodeArgs& a, hipStream_t st) {
#define CALL(d, k, v) launch_split_g<d, k, v>(gq, a, st)
  if (D == 128) KVARN_FOR_VB(128, KB, vb, CALL);
  else KVARN_FOR_VB(256, KB, vb, CALL);
#undef CALL
  return hipGetLastError();
}

template <int KB>
static int resident_split_kb(int D, int vb, int gq, int dev) {
  int r = 0;
#define CALL(d, k, v) r = resident_g<d, k, v>(gq, dev)
  if (D == 128) KVARN_FOR_VB(128, KB, vb, CALL);
  else KVARN_FOR_VB(256, KB, vb, CALL);
#undef CALL
  return r;
}

}  // namespace kvarn
