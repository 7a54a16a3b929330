// KVarN chunked-prefill attention on gfx950: the queries of a prefill chunk
// (the last C cached positions of each request) attend causally over the
// cache as it holds them -- the exact fp16 sink and tail, and the sealed
// groups read directly from their records -- on fp16 MFMA with fp32
// accumulation ["KVarN KV Cache: Implementation and Benchmarks"
// (anbeeld.com), §2.1 "Sink, Body, And Tail": attention paths read the
// records; §1 "Where KVarN Comes From": attention over a record runs in the
// rotated frame, and the result is rotated back once].
//
// Workgroup = NW waves = 16 NW query rows of one (request, KV head): row
// r = position-in-block * GQ + head, so the GQ query heads of a KV head share
// every key tile staged in LDS.  Wave w owns rows 16w .. 16w+15; lane l
// (n = l % 16, G = l / 16) owns row 16w + n.  With NW = 8 (D 128, when the
// grid still has a workgroup for every CU) waves 0-3 stage the K half of
// each next tile and waves 4-7 its V half, so a wave stages one 64-code item
// per tile for twice the query rows of a four-wave workgroup.  With NW = 4
// (D 256, whose working set needs one wave per SIMD, and short chunks)
// every wave stages its items of both halves.  The products are taken
// transposed -- S^T = K q^T and O^T = V^T P^T -- so an MFMA result lane
// holds one query row: logits, softmax state and output stay in registers
// with no LDS transposition (v_mfma_f32_16x16x32_f16 lane layout, checked on
// the device: A lane l holds row l%16, k = 8(l/16)..+7; B lane l holds
// column l%16, same k; C lane l holds column l%16, rows 4(l/16)..+3).
//
// Tiles, in position order: the sink, the sealed groups, the tail, each 128
// tokens at most, up to the block's last row.
//   * record tile (rotated frame): the codes minus the mid level, exact in
//     fp16, are the A operand; the query operand is q~ = q_r * c^K, an fp32
//     value split into fp16 hi + lo (two MFMAs), so the logit
//     s^K_t * (q~ . (code - mid)) keeps fp32 accuracy; PV takes the weights
//     w = p * s^V_t, split the same way, against the V codes and scales by
//     c^V_j.
//   * exact tile (original frame): fp16 q against fp16 K rows, one MFMA
//     (products of fp16 values are exact in fp32); PV as for a record.
// The output accumulator is rotated (H / sqrt(D), its own inverse) whenever
// the frame changes, so it leaves the kernel in the original frame.
//
// Pipeline: while a tile is computed, the next record's codes and scales are
// already loading into registers; its K half is decoded into LDS after the
// QK step, its V half after the PV step (two barriers per tile).
//
// Codes are turned into fp16 two at a time: 2c is placed in the mantissa of
// 512 (fp16 spacing 1/2 in [512, 1024)) and 512 + mid is subtracted with one
// packed fp16 add, exact.  For 2/4/8-bit codes a dword of codes yields pairs
// (i, i + B/2) of each B = 32/bits block, so tile rows hold their codes in
// that order; the query operand, the scales and the K tile's token rows are
// permuted to match (exact tiles are staged in the same orders).
#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace kvarn {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
constexpr float kPaLog2e = 1.4426950408889634f;

// LDS tiles: row pitches of 8 (mod 64) dwords make the MFMA operand reads
// (lanes 16G + n: row n, 16-byte column G) conflict-free -- a 128-bit read
// is served for lanes {0-7, 16-23}, {8-15, 24-31}, ... together -- and the
// 128-bit row writes of the staging are conflict-free when lanes
// {4j .. 4j+3, 4j+8 .. 4j+11} (served together) write rows that differ mod 8,
// which write_row() arranges.
// Staged query rows (fp32, pitch QP = 8 mod 64 dwords) hold the value of
// K-tile column position p = 32 s + 8 G + 4 h + e at 32 s + 16 h + 4 G + e,
// so that lane 16 G + n reads its 8 values of step s as two conflict-free
// 128-bit reads.  Four-wave workgroups stage them over the K and V tiles
// and keep them in registers; eight-wave ones keep them in LDS (KEEPQ).
template <int D, bool KEEPQ>
struct PaSmem {
  static constexpr int KP = D + 16;    // K tile: 128 token rows, pitch in halves
  static constexpr int VP = 128 + 16;  // V tile: D channel rows of 128 token positions
  static constexpr int QP = D + 8;     // staged query rows (fp32)
  static_assert(128 * QP * 4 <= 128 * KP * 2 + D * VP * 2, "staged queries fit the K and V tiles");
  alignas(16) float q[KEEPQ ? 128 * QP : 4];   // kept query rows
  alignas(16) _Float16 k[128 * KP];
  alignas(16) _Float16 v[D * VP];
  alignas(16) float sk[128];   // per K tile row: s^K of its token
  alignas(16) float sv[128];   // per K tile row: s^V of its token / 2^eV
  alignas(16) float ck[2 * D]; // per K tile column: c^K of its channel / 2^eK (two tiles' worth)
  alignas(16) float cv[D];     // per channel: c^V * 2^eV
  float qinv[128];             // per row: inverse power-of-two scale of the staged query
  float kscale[2];             // 2^eK of the record tiles in the two c^K buffers
  float vscale;                // 2^eV of the staged record tile
};

// ---- orders -------------------------------------------------------------
// Block size B of the pair order of a code width (2 = natural order).
__device__ __forceinline__ int perm_block(int bits) { return bits == 2 ? 16 : bits == 4 ? 8 : bits == 8 ? 4 : 2; }
// Position p of a tile row -> index of the code it holds, and back.
__device__ __forceinline__ int pos_to_code(int p, int B) {
  return (p & -B) | ((p & (B - 1)) >> 1) | ((p & 1) * (B >> 1));
}
__device__ __forceinline__ int code_to_pos(int c, int B) {
  const int h = B >> 1;
  return (c & -B) | ((c & (h - 1)) << 1) | ((c & h) ? 1 : 0);
}
// Slot of K-tile column position p in a staged query row (see PaSmem).
__device__ __forceinline__ int q_slot(int p) { return (p & ~31) | ((p & 4) << 2) | ((p & 24) >> 1) | (p & 3); }
// K tile row r <-> V tile position p, within 32-token blocks: row bits
// (i: 2, G: 2, h: 1) are position bits (i: 2, h: 1, G: 2).  A QK result lane
// then holds, for PV step u, the weights of positions 32u + 8G .. +7: its B
// operand, with no data movement.
__device__ __forceinline__ int vpos_to_krow(int p) { return (p & ~31) | (p & 3) | ((p & 4) << 2) | ((p & 24) >> 1); }
__device__ __forceinline__ int krow_to_vpos(int r) { return (r & ~31) | (r & 3) | ((r & 16) >> 2) | ((r & 12) << 1); }

// Power of two that brings x > 0 into [2^11, 2^12) (1 for x = 0), and its inverse.
__device__ __forceinline__ float pow2_scale(float x, float& inv) {
  if (!(x > 0.f)) {
    inv = 1.f;
    return 1.f;
  }
  int e;
  (void)frexpf(x, &e);   // x = m 2^e, m in [0.5, 1)
  inv = ldexpf(1.f, e - 12);
  return ldexpf(1.f, 12 - e);
}

// Maximum of v over lanes l, l^16, l^32, l^48 (the four lane groups).
__device__ __forceinline__ float max_over_groups(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float dpp_pair_f(float x, int st) {
  const int v = __float_as_int(x);
  int o;
  if (st == 1) {
    o = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if (st == 2) {
    o = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if (st == 4) {
    o = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0, 2
    o = __builtin_amdgcn_update_dpp(o, v, 0x114, 0xF, 0xA, false);  // row_shr:4, banks 1, 3
  } else {
    o = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true);  // row_ror:8
  }
  return __int_as_float(o);
}

// Rotate fp16 rows of D channels by H_D / sqrt(D) (natural-order Sylvester)
// in fp32: thread (row, 64-channel chunk), NT = D/64 adjacent threads per
// row; butterflies over the six low channel bits in registers, over the
// chunk bits across lanes.  x holds the 64 values of the thread's chunk.
template <int D>
__device__ __forceinline__ void rotate64(float (&x)[64], int chunk) {
#pragma unroll
  for (int st = 1; st < 64; st <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (!(i & st)) {
        const float a = x[i], b = x[i + st];
        x[i] = a + b;
        x[i + st] = a - b;
      }
    }
  }
#pragma unroll
  for (int st = 1; st < D / 64; st <<= 1) {
    const bool upper = chunk & st;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float o = dpp_pair_f(x[i], st);
      x[i] = upper ? o - x[i] : x[i] + o;
    }
  }
  const float rs = D == 128 ? 0.08838834764831845f : 0.0625f;
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] *= rs;
}

__device__ __forceinline__ void load64h(float (&x)[64], const __half* p, bool valid) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 w = valid ? reinterpret_cast<const uint4*>(p)[k] : make_uint4(0, 0, 0, 0);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * k + 2 * e] = h2f((uint16_t)(ws[e] & 0xFFFFu));
      x[8 * k + 2 * e + 1] = h2f((uint16_t)(ws[e] >> 16));
    }
  }
}

__device__ __forceinline__ v8h ld8(const _Float16* p) { return *reinterpret_cast<const v8h*>(p); }

// Tile row written by thread index x in the staging (bits 2 and 3 swapped).
__device__ __forceinline__ int write_row(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// Output rotation by H_D / sqrt(D) over the C-layout channels 16 ct + 4 G + i
// of one query row: butterflies over i and ct in registers, over G across
// the lane groups.
template <int NCT>
__device__ __forceinline__ void rotate_out(v4f (&o)[NCT], int G) {
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const float a0 = o[c][0] + o[c][1], a1 = o[c][0] - o[c][1];
    const float a2 = o[c][2] + o[c][3], a3 = o[c][2] - o[c][3];
    o[c] = v4f{a0 + a2, a1 + a3, a0 - a2, a1 - a3};
  }
#pragma unroll
  for (int st = 1; st < NCT; st <<= 1) {
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      if (!(c & st)) {
        const v4f u = o[c], v = o[c + st];
        o[c] = u + v;
        o[c + st] = u - v;
      }
    }
  }
#pragma unroll
  for (int gb = 1; gb < 4; gb <<= 1) {
    const bool upper = G & gb;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = o[c][i];
        const float y = __shfl_xor(x, 16 * gb);
        o[c][i] = upper ? y - x : x + y;
      }
  }
  const float rs = NCT == 8 ? 0.08838834764831845f : 0.0625f;
#pragma unroll
  for (int c = 0; c < NCT; ++c) o[c] *= rs;
}

// ---- code decode -----------------------------------------------------------
// x holds 2c0 in bits 1.. and 2c1 in bits 17..: (512 + c0, 512 + c1) - (512 + mid).
__device__ __forceinline__ uint32_t code_pair(uint32_t x, v2h off) {
  const v2h h = __builtin_bit_cast(v2h, x | 0x60006000u) + off;
  return __builtin_bit_cast(uint32_t, h);
}
// (x & m) | c in one instruction: VOP3 takes no literal operand and one
// scalar operand on this target, so m sits in a vector and c in a scalar
// register (the compiler would emit a separate AND and OR with literals).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "s"(c));
  return r;
}
__device__ __forceinline__ uint32_t biased_code_pair(uint32_t x, v2h off) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, x) + off);
}

// 64 codes of BITS bits (a little-endian bit stream in w) -> 64 fp16
// (code - mid) at dst, in the width's pair order.
template <int BITS>
__device__ __forceinline__ void decode_item(const uint32_t* w, _Float16* dst) {
  constexpr float MID = 0.5f * ((1 << BITS) - 1);
  const v2h off = {(_Float16)(-512.f - MID), (_Float16)(-512.f - MID)};
  uint32_t out[32];
  if constexpr (BITS == 2 || BITS == 4 || BITS == 8) {
    constexpr int HALF = 16 / BITS;   // output dwords per input dword
    constexpr uint32_t M = ((1u << BITS) - 1) << 1;
    constexpr uint32_t MASK = M | (M << 16);
#pragma unroll
    for (int d = 0; d < 2 * BITS; ++d)
#pragma unroll
      for (int m = 0; m < HALF; ++m) {
        const uint32_t x = m == 0 ? (w[d] << 1) : (w[d] >> (BITS * m - 1));
        out[HALF * d + m] = biased_code_pair(and_or(x, MASK, 0x60006000u), off);
      }
  } else {
    constexpr uint32_t M = (1u << BITS) - 1;
#pragma unroll
    for (int o = 0; o < 32; ++o) {
      uint32_t c[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bit = BITS * (2 * o + h), wi = bit >> 5, sh = bit & 31;
        c[h] = sh + BITS <= 32 ? (w[wi] >> sh) & M : __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & M;
      }
      out[o] = code_pair((c[0] << 1) | (c[1] << 17), off);
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    reinterpret_cast<uint4*>(dst)[k] = make_uint4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
}

template <int MAXB>
__device__ __forceinline__ void decode_item_rt(const uint32_t (&w)[2 * MAXB], int bits, _Float16* dst) {
  switch (bits) {
    case 2: decode_item<2>(w, dst); break;
    case 3: decode_item<3>(w, dst); break;
    case 4: decode_item<4>(w, dst); break;
    default:
      if constexpr (MAXB >= 8) {
        if (bits == 5) decode_item<5>(w, dst);
        else if (bits == 6) decode_item<6>(w, dst);
        else decode_item<8>(w, dst);
      }
      break;
  }
}

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) int32_t ConstI32;   // read-only: scalar loads

// Buffer resource over one record (`bytes` bytes at a wave-uniform address):
// loads past its end return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const uint8_t* rec, int bytes) {
  const uint64_t addr = reinterpret_cast<uint64_t>(rec);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 8 * MAXB bytes from byte offset `off` of a record: the 8 * bits bytes of a
// 64-code item (8-byte aligned) and whatever follows it.  A fixed number of
// loads with no width test: loads under a width test get moved down to
// their use, which would undo the prefetch.
template <int MAXB>
__device__ __forceinline__ void load_item(uint32_t (&w)[2 * MAXB], __amdgpu_buffer_rsrc_t r, int off) {
#pragma unroll
  for (int k = 0; k < MAXB; ++k) {
    const v2u x = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8 * k, 0, 0);
    w[2 * k] = x[0];
    w[2 * k + 1] = x[1];
  }
}

}  // namespace

template <int D, int GQ, int MAXB, int NW>
__global__ __launch_bounds__(64 * NW, (D == 128 && NW == 4) ? 2 : 1) void prefill_attn_kernel(PrefillAttnArgs a) {
  static_assert(NW == 4 || (NW == 8 && D == 128), "four waves, or eight at head dimension 128");
  constexpr bool SPLIT = NW == 8;  // K and V staging split between the wave halves
  // MFMA A operands read a group ahead: eight-wave workgroups, and D 256,
  // where one wave per SIMD has no other wave to cover its LDS latency.
  constexpr bool READ_AHEAD = SPLIT || D == 256;
  __shared__ PaSmem<D, SPLIT> sm;
  constexpr int ROWS = 16 * NW;   // query rows
  constexpr int KS = D / 32;      // MFMA k-steps over the channels
  constexpr int NCT = D / 16;     // output channel tiles
  constexpr int POS = ROWS / GQ;  // positions per workgroup
  constexpr int NI = D / 128;     // K or V items of 64 codes per thread
  constexpr int KP = PaSmem<D, SPLIT>::KP, VP = PaSmem<D, SPLIT>::VP, QP = PaSmem<D, SPLIT>::QP;
  // Eight-wave workgroups branch on the wave half: a scalar wave index keeps
  // those branches (and the loads inside them) uniform.
  const int w = SPLIT ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
  const bool vrole = SPLIT && w >= NW / 2;   // stages V items only (else K items); wave-uniform
  int tid = threadIdx.x, l = tid & 63;   // re-derived per tile (see the tile loop)
  const int G = l >> 4, n = l & 15;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int nseq = a.c.seq_len[b];
  const int C = a.chunk;
  const int64_t bh = (int64_t)b * a.c.hkv + kvh;
  const int kb = a.k_bits, vb = a.v_bits;
  const int Bk = perm_block(kb), Bv = perm_block(vb);
  const float qk_scale = a.scale * kPaLog2e;
  auto row_pos = [&](int r) {   // position of workgroup row r, or -1
    const int i = blockIdx.x * POS + r / GQ;
    const int p = nseq - C + i;
    return (i < C && p >= 0) ? p : -1;
  };
  auto krow_of_token = [&](int t) { return vpos_to_krow(code_to_pos(t, Bv)); };
  auto token_of_krow = [&](int r) { return pos_to_code(krow_to_vpos(r), Bv); };
  int pmax = -1, pmin = 0x7fffffff;
#pragma unroll 1
  for (int r = 0; r < ROWS; ++r) {
    const int p = row_pos(r);
    if (p >= 0) {
      pmax = max(pmax, p);
      pmin = min(pmin, p);
    }
  }
  if (pmax < 0) return;   // no row of this block is in the chunk (uniform)

  const int r_lane = 16 * w + n;
  const int prow = row_pos(r_lane);
  const __half* qrow =
      a.q + (((int64_t)b * C + blockIdx.x * POS + r_lane / GQ) * a.hq + kvh * GQ + r_lane % GQ) * D;

  // ---- queries: rotated, times softmax_scale * log2(e), times a per-row
  // power of two that puts the row's largest magnitude in [2^11, 2^12)
  // (fp32 in LDS, each channel at the slot of its K-tile column position in
  // the K width's pair order); read as the B operand.
  float* const qs = SPLIT ? sm.q : reinterpret_cast<float*>(sm.k);
  {
    constexpr int NT = D / 64;
#pragma unroll 1
    for (int it = tid; it < ROWS * NT; it += 64 * NW) {
      const int r = it / NT, chunk = it % NT;
      const int p = row_pos(r);
      float x[64];
      load64h(x,
              a.q + (((int64_t)b * C + (p >= 0 ? blockIdx.x * POS + r / GQ : 0)) * a.hq + kvh * GQ + r % GQ) * D +
                  64 * chunk,
              p >= 0);
      rotate64<D>(x, chunk);   // the NT threads of a row are adjacent lanes
      float mx = 0.f;
#pragma unroll
      for (int k = 0; k < 64; ++k) mx = fmaxf(mx, fabsf(x[k]));
      mx = fmaxf(mx, dpp_pair_f(mx, 1));
      if (NT == 4) mx = fmaxf(mx, dpp_pair_f(mx, 2));
      float inv;
      const float sc = pow2_scale(mx * qk_scale, inv) * qk_scale;
#pragma unroll
      for (int k = 0; k < 64; ++k) qs[r * QP + q_slot(code_to_pos(64 * chunk + k, Bk))] = x[k] * sc;
      if (chunk == 0) sm.qinv[r] = inv;
    }
  }
  lds_barrier();
  float qr[KS][8];   // the lane's query row, in registers for a tile's use
  auto read_query = [&]() {
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4f x = *reinterpret_cast<const v4f*>(qs + r_lane * QP + 32 * s + 16 * h + 4 * G);
#pragma unroll
        for (int e = 0; e < 4; ++e) qr[s][4 * h + e] = x[e];
      }
  };
  if (!SPLIT) read_query();
  const float qinv = sm.qinv[r_lane];
  if (!SPLIT) lds_barrier();   // the staged queries are read; the K and V tiles are free

  // ---- staging --------------------------------------------------------------
  // Exact tile: `count` fp16 rows [128][D] at src (rows past count are zero),
  // by threads [t0, t0 + nt) of the workgroup.
  auto stage_k_exact = [&](const __half* __restrict__ src, int count, int t0, int nt) {
#pragma unroll 4
    for (int idx = tid - t0; idx < 128 * D / 8; idx += nt) {
      const int r = write_row(idx & 127), c8 = idx >> 7;
      const int t = token_of_krow(r);
      const uint4 x = t < count ? *reinterpret_cast<const uint4*>(src + (size_t)t * D + 8 * c8) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(sm.k + r * KP + 8 * c8) = x;
    }
    for (int t = tid - t0; t < 128; t += nt) {
      sm.sk[t] = 1.f;
      sm.sv[t] = 1.f;
    }
  };
  auto stage_v_exact = [&](const __half* __restrict__ src, int count, int t0, int nt) {
#pragma unroll 4
    for (int idx = tid - t0; idx < 128 * D / 8; idx += nt) {
      const int t = idx % 128, c8 = idx / 128;
      const uint4 x = t < count ? *reinterpret_cast<const uint4*>(src + (size_t)t * D + 8 * c8) : make_uint4(0, 0, 0, 0);
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
      const int p = code_to_pos(t, Bv);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sm.v[(8 * c8 + e) * VP + p] = __builtin_bit_cast(_Float16, (uint16_t)(xs[e >> 1] >> (16 * (e & 1))));
    }
    for (int j = tid - t0; j < D; j += nt) sm.cv[j] = 1.f;
  };

  // Record tile: registers of the next record: codes of this thread's items
  // (set 0: K items, or V items in the V waves of a split workgroup; set 1:
  // V items when every wave stages both halves) and the scale dwords of this
  // wave's scale vector (role 0 s^K, 1 c^K, 2 s^V: waves 0-2; role 3 c^V:
  // wave 4 of a split workgroup, else wave 3).
  constexpr int NSETS = SPLIT ? 1 : 2;
  uint32_t rc[NSETS][NI][2 * MAXB], rs[NI];
  const int kcode = 16 * D * kb, vcode = 16 * D * vb, vrec = a.c.rec_k_bytes;
  // Tile-invariant item placement of this thread (kept in registers), with
  // it = its index among the 256 threads that stage the same half: K item =
  // tile row write_row(it % 128), holding token token_of_krow(that row),
  // 64-channel chunk it / 128; V item = channel write_row(it % D), 64-token
  // chunk it / D.  Byte offsets within the record, element offsets in LDS.
  int coff[NSETS][NI], cdst[NSETS][NI];
#pragma unroll
  for (int set = 0; set < NSETS; ++set) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int it = ((int)threadIdx.x & 255) + 256 * i;
      if (!(vrole || set == 1)) {
        const int r = write_row(it & 127);
        coff[set][i] = (token_of_krow(r) * (D / 64) + (it >> 7)) * 8 * kb;
        cdst[set][i] = r * KP + 64 * (it >> 7);
      } else {
        const int jv = write_row(it & (D - 1));
        coff[set][i] = vrec + (2 * jv + it / D) * 8 * vb;
        cdst[set][i] = jv * VP + 64 * (it / D);
      }
    }
  }
  const int role = SPLIT ? (w < 3 ? w : w == 4 ? 3 : -1) : w;
  const int soff = (role < 2 ? kcode : vrec + vcode) + 4 * ((role & 1) ? 64 + l : l);
  auto issue_record = [&](const uint8_t* __restrict__ rec) {
    const __amdgpu_buffer_rsrc_t r = record_rsrc(rec, (int)a.c.group_bytes);
#pragma unroll
    for (int set = 0; set < NSETS; ++set)
#pragma unroll
      for (int i = 0; i < NI; ++i) load_item<MAXB>(rc[set][i], r, coff[set][i]);
    if (role >= 0) {
      rs[0] = __builtin_amdgcn_raw_buffer_load_b32(r, soff, 0, 0);
      if (NI > 1) rs[NI - 1] = __builtin_amdgcn_raw_buffer_load_b32(r, soff + 256, 0, 0);   // c^K / c^V waves
    }
  };
  // Role 1: c^K of the record in rs, normalized by the power of two of its
  // maximum so that q~ stays below 2^12, into c^K buffer buf.
  auto stage_ck = [&](int buf) {
    float x[2 * NI];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      x[2 * i] = h2f((uint16_t)(rs[i] & 0xFFFFu));
      x[2 * i + 1] = h2f((uint16_t)(rs[i] >> 16));
      mx = fmaxf(mx, fmaxf(x[2 * i], x[2 * i + 1]));
    }
    mx = wave_max_f(mx);
    int e;
    (void)frexpf(mx, &e);
    const float down = ldexpf(1.f, -e);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) sm.ck[buf * D + code_to_pos(2 * (l + 64 * i) + h, Bk)] = x[2 * i + h] * down;
    if (l == 0) sm.kscale[buf] = ldexpf(1.f, e);
  };
  auto stage_k_record = [&]() {   // K-staging waves
#pragma unroll
    for (int i = 0; i < NI; ++i) decode_item_rt<MAXB>(rc[0][i], kb, sm.k + cdst[0][i]);
    if (role == 0) {
      sm.sk[krow_of_token(2 * l)] = h2f((uint16_t)(rs[0] & 0xFFFFu));
      sm.sk[krow_of_token(2 * l + 1)] = h2f((uint16_t)(rs[0] >> 16));
    } else if (role == 1) {
      if (!SPLIT) stage_ck(0);   // eight-wave workgroups stage c^K a window earlier
    } else if (role == 2) {
      // s^V, normalized by the power of two of its maximum so that
      // w = p s^V stays below 1
      const float x0 = h2f((uint16_t)(rs[0] & 0xFFFFu)), x1 = h2f((uint16_t)(rs[0] >> 16));
      const float mx = wave_max_f(fmaxf(x0, x1));
      int e;
      (void)frexpf(mx, &e);
      const float down = ldexpf(1.f, -e);
      sm.sv[krow_of_token(2 * l)] = x0 * down;
      sm.sv[krow_of_token(2 * l + 1)] = x1 * down;
      if (l == 0) sm.vscale = ldexpf(1.f, e);
    }
  };
  auto stage_v_record = [&]() {   // V-staging waves
#pragma unroll
    for (int i = 0; i < NI; ++i) decode_item_rt<MAXB>(rc[NSETS - 1][i], vb, sm.v + cdst[NSETS - 1][i]);
    if (role == 3) {
      const float up = sm.vscale;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        sm.cv[2 * (l + 64 * i)] = h2f((uint16_t)(rs[i] & 0xFFFFu)) * up;
        sm.cv[2 * (l + 64 * i) + 1] = h2f((uint16_t)(rs[i] >> 16)) * up;
      }
    }
  };

  // ---- tiles: 0 = sink, 1 .. n_rec = records (group t - 1), then the tail
  const int n_groups = nseq > kSink ? min((nseq - kSink) / kGroup, a.c.max_groups) : 0;
  const int n_rec = pmax >= kSink ? min(n_groups, (pmax - kSink) / kGroup + 1) : 0;
  const int tail_base = kSink + kGroup * n_groups;
  const bool has_tail = n_rec == n_groups && nseq > tail_base && tail_base <= pmax;
  const int T = 1 + n_rec + (has_tail ? 1 : 0);
  const int tail_count = min(nseq - tail_base, kGroup);
  const int32_t* table = a.c.map.table;
  // Block-table entry of the next record (scalar loads, a tile ahead).
  int ent = (table && n_rec > 0) ? *(ConstI32*)(table + (int64_t)b * a.c.max_groups) : 0;

  stage_k_exact(a.c.sink_k + bh * kGroup * D, min(nseq, kSink), 0, 64 * NW);
  stage_v_exact(a.c.sink_v + bh * kGroup * D, min(nseq, kSink), 0, 64 * NW);
  lds_barrier();

  PhaseClock pc;   // trace build only: cycles per phase, summed over the tiles
  phase_start(pc);
  float m_run = -INFINITY, l_run = 0.f;
  v4f o[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) o[c] = v4f{0.f, 0.f, 0.f, 0.f};
  bool rotated = false;   // frame of o

  // ---- the phases of a tile, for one wave --------------------------------
  v8h bhi[KS], blo[KS];   // QK B operand: the query (hi + lo)
  float lg[8][4];         // QK results, then the softmax weights
  float f;                // logit scale to log2 units
  v8h bwh[4], bwl[4];     // PV B operands: w = p * s^V (hi + lo) for positions 32 u + 8 G + e

  // Exact tile: the fp16 query rows as the B operand.  Loaded and waited for
  // before the next record's loads are issued: the load counter completes in
  // order, so a wait for them issued later would also wait for that whole
  // prefetch.
  auto load_exact_query = [&]() {
    uint4 x[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      x[s] = prow >= 0 ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * G) : make_uint4(0, 0, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      asm volatile("" : "+v"(x[s].x), "+v"(x[s].y), "+v"(x[s].z), "+v"(x[s].w));   // ready here
      bhi[s] = __builtin_bit_cast(v8h, x[s]);
      blo[s] = v8h{};   // one code path for both kinds: the low product adds zero
    }
  };
  // Issues this thread's loads of tile t + 1 when it is a record; returns
  // whether tile t + 1 has storage.
  auto issue_next = [&](int t) {
    bool np = t + 1 < T;
    if (t + 1 <= n_rec) {
      const int g = t;
      int64_t off;
      if (!table) {
        off = (bh * a.c.max_groups + g) * a.c.group_bytes;
      } else {
        off = (ent >= 0 && ent < a.c.map.num_blocks) ? ((int64_t)ent * a.c.hkv + kvh) * a.c.group_bytes : -1;
        if (g + 1 < n_rec) ent = *(ConstI32*)(table + (int64_t)b * a.c.max_groups + g + 1);
      }
      np = off >= 0;
      if (np) issue_record(a.c.records + off);
    }
    return np;
  };
  // Record tile: the query operand q~ = q_r c^K (c^K from buffer buf),
  // split into fp16 hi + lo; returns the logit scale to log2 units.
  auto record_operand = [&](int buf) {
    if (SPLIT) read_query();   // kept in LDS: 32 registers fewer across the steps
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const v4f c0 = *reinterpret_cast<const v4f*>(sm.ck + buf * D + 32 * s + 8 * G);
      const v4f c1 = *reinterpret_cast<const v4f*>(sm.ck + buf * D + 32 * s + 8 * G + 4);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float x0 = qr[s][e] * (e < 4 ? c0[e] : c1[e - 4]);
        const float x1 = qr[s][e + 1] * (e < 4 ? c0[e + 1] : c1[e - 3]);
        const float h0 = __uint_as_float(__float_as_uint(x0) & 0xFFFFE000u);   // fp16-exact high part
        const float h1 = __uint_as_float(__float_as_uint(x1) & 0xFFFFE000u);
        const auto ph = __builtin_amdgcn_cvt_pkrtz(h0, h1);
        const auto pl = __builtin_amdgcn_cvt_pkrtz(x0 - h0, x1 - h1);
        bhi[s][e] = ph[0];
        bhi[s][e + 1] = ph[1];
        blo[s][e] = pl[0];
        blo[s][e + 1] = pl[1];
      }
    }
    return qinv * sm.kscale[buf];
  };
  // QK^T with the query operand in bhi / blo: logits of the lane's row for K
  // tile rows 16 tt + 4 G + i.
  auto qk_products = [&]() {
    if constexpr (READ_AHEAD) {
      // Two token tiles at a time (independent MFMA chains), in groups of two
      // k-steps: the next group's A operands are read from LDS before this
      // group's eight products are issued, so a wave covers its own LDS
      // latency (in an eight-wave workgroup, half the waves stage meanwhile;
      // at D 256 a wave has its SIMD to itself; a four-wave workgroup at
      // D 128 has no registers to spare for it).
      constexpr int NG = 4 * KS / 2;   // groups: 4 token-tile pairs x KS / 2
      v8h A[2][4];
      auto load_a = [&](v8h* dst, int gi) {
        const int tp = 2 * (gi / (KS / 2)), s0 = 2 * (gi % (KS / 2));
        const _Float16* kr0 = sm.k + (16 * tp + n) * KP + 8 * G;
        dst[0] = ld8(kr0 + 32 * s0);
        dst[1] = ld8(kr0 + 16 * KP + 32 * s0);
        dst[2] = ld8(kr0 + 32 * s0 + 32);
        dst[3] = ld8(kr0 + 16 * KP + 32 * s0 + 32);
      };
      load_a(A[0], 0);
      v4f acc0, acc1;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        if (gi + 1 < NG) load_a(A[(gi + 1) & 1], gi + 1);
        __builtin_amdgcn_sched_barrier(0);   // the next group's reads stay ahead of this group's products
        const int tp = 2 * (gi / (KS / 2)), s0 = 2 * (gi % (KS / 2));
        if (s0 == 0) acc0 = acc1 = v4f{0.f, 0.f, 0.f, 0.f};
        const v8h* a = A[gi & 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h], bhi[s0 + h], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h + 1], bhi[s0 + h], acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h], blo[s0 + h], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h + 1], blo[s0 + h], acc1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (s0 + 2 == KS) {
          const v4f sk0 = *reinterpret_cast<const v4f*>(sm.sk + 16 * tp + 4 * G);
          const v4f sk1 = *reinterpret_cast<const v4f*>(sm.sk + 16 * tp + 16 + 4 * G);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lg[tp][i] = acc0[i] * sk0[i];
            lg[tp + 1][i] = acc1[i] * sk1[i];
          }
        }
      }
    } else {
#pragma unroll
      for (int tp = 0; tp < 8; tp += 2) {   // two token tiles at a time: independent MFMA chains
        v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const _Float16* kr0 = sm.k + (16 * tp + n) * KP + 8 * G;
        const _Float16* kr1 = kr0 + 16 * KP;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const v8h a0 = ld8(kr0 + 32 * s), a1 = ld8(kr1 + 32 * s);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bhi[s], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bhi[s], acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, blo[s], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, blo[s], acc1, 0, 0, 0);
        }
        const v4f sk0 = *reinterpret_cast<const v4f*>(sm.sk + 16 * tp + 4 * G);
        const v4f sk1 = *reinterpret_cast<const v4f*>(sm.sk + 16 * tp + 16 + 4 * G);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lg[tp][i] = acc0[i] * sk0[i];
          lg[tp + 1][i] = acc1[i] * sk1[i];
        }
      }
    }
  };
  // Online softmax of the lane's row (its 128 tokens span the four lane
  // groups) and the PV operands; tiles below every row of the block and
  // complete need no mask.
  auto softmax = [&](int base, int count) {
    const bool full = __builtin_amdgcn_readfirstlane((int)(count == kGroup && base + kGroup - 1 <= pmin)) != 0;
    float alpha, m_new, ps = 0.f;
    if (full) {
      float mx = lg[0][0];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, lg[tt][i]);
      m_new = fmaxf(m_run, max_over_groups(mx) * f);
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lg[tt][i] = __builtin_amdgcn_exp2f(fmaf(lg[tt][i], f, -m_new));
          ps += lg[tt][i];
        }
    } else {
      // causal and length mask: token of K tile row 16 tt + 4 G + i
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = token_of_krow(16 * tt + 4 * (l >> 4) + i);
          if (!(tok < count && base + tok <= prow)) lg[tt][i] = -INFINITY;
        }
      float mx = lg[0][0];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, lg[tt][i]);
      m_new = fmaxf(m_run, max_over_groups(mx) * f);
      alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lg[tt][i] = lg[tt][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(lg[tt][i], f, -m_new));
          ps += lg[tt][i];
        }
    }
    l_run = fmaf(l_run, alpha, xor32_sum(xor16_sum(ps)));
    m_run = m_new;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const v4f sv4 = *reinterpret_cast<const v4f*>(sm.sv + 16 * tt + 4 * G);
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float x0 = lg[tt][i] * sv4[i], x1 = lg[tt][i + 1] * sv4[i + 1];
        const float h0 = __uint_as_float(__float_as_uint(x0) & 0xFFFFE000u);
        const float h1 = __uint_as_float(__float_as_uint(x1) & 0xFFFFE000u);
        const auto ph = __builtin_amdgcn_cvt_pkrtz(h0, h1);
        const auto pl = __builtin_amdgcn_cvt_pkrtz(x0 - h0, x1 - h1);
        const int e = 4 * (tt & 1) + i;
        bwh[tt >> 1][e] = ph[0];
        bwh[tt >> 1][e + 1] = ph[1];
        bwl[tt >> 1][e] = pl[0];
        bwl[tt >> 1][e + 1] = pl[1];
      }
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int c = 0; c < NCT; ++c) o[c] *= alpha;
    }
  };
  // PV: O^T += V^T w^T, channel tiles of 16, token steps of 32.
  auto pv = [&](bool exact) {
    if (rotated == exact) {   // frame change
      rotate_out<NCT>(o, G);
      rotated = !exact;
    }
    if constexpr (READ_AHEAD) {
      // Two channel tiles at a time, in groups of two token steps, the next
      // group's A operands read ahead as in QK.
      constexpr int NG = NCT / 2 * 2;   // groups: NCT / 2 channel-tile pairs x 2
      v8h A[2][4];
      auto load_a = [&](v8h* dst, int gi) {
        const int cp = 2 * (gi / 2), u0 = 2 * (gi % 2);
        const _Float16* vr0 = sm.v + (16 * cp + n) * VP + 8 * G;
        dst[0] = ld8(vr0 + 32 * u0);
        dst[1] = ld8(vr0 + 16 * VP + 32 * u0);
        dst[2] = ld8(vr0 + 32 * u0 + 32);
        dst[3] = ld8(vr0 + 16 * VP + 32 * u0 + 32);
      };
      load_a(A[0], 0);
      v4f acc0, acc1;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        if (gi + 1 < NG) load_a(A[(gi + 1) & 1], gi + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int cp = 2 * (gi / 2), u0 = 2 * (gi % 2);
        if (u0 == 0) acc0 = acc1 = v4f{0.f, 0.f, 0.f, 0.f};
        const v8h* a = A[gi & 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h], bwh[u0 + h], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h + 1], bwh[u0 + h], acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h], bwl[u0 + h], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2 * h + 1], bwl[u0 + h], acc1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (u0 == 2) {
          const v4f cv0 = *reinterpret_cast<const v4f*>(sm.cv + 16 * cp + 4 * G);
          const v4f cv1 = *reinterpret_cast<const v4f*>(sm.cv + 16 * cp + 16 + 4 * G);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[cp][i] = fmaf(acc0[i], cv0[i], o[cp][i]);
            o[cp + 1][i] = fmaf(acc1[i], cv1[i], o[cp + 1][i]);
          }
        }
      }
    } else {
#pragma unroll
      for (int cp = 0; cp < NCT; cp += 2) {   // two channel tiles at a time
        v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const _Float16* vr0 = sm.v + (16 * cp + n) * VP + 8 * G;
        const _Float16* vr1 = vr0 + 16 * VP;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const v8h a0 = ld8(vr0 + 32 * u), a1 = ld8(vr1 + 32 * u);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bwh[u], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bwh[u], acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bwl[u], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bwl[u], acc1, 0, 0, 0);
        }
        const v4f cv0 = *reinterpret_cast<const v4f*>(sm.cv + 16 * cp + 4 * G);
        const v4f cv1 = *reinterpret_cast<const v4f*>(sm.cv + 16 * cp + 16 + 4 * G);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[cp][i] = fmaf(acc0[i], cv0[i], o[cp][i]);
          o[cp + 1][i] = fmaf(acc1[i], cv1[i], o[cp + 1][i]);
        }
      }
    }
  };
  // Staging of tile u >= 1 (the tail, or a record whose loads were issued a
  // tile ahead): K half by the K-staging threads, V half by the V-staging ones.
  auto stage_k_tile = [&](int u, bool pres) {
    if (has_tail && u == T - 1)
      stage_k_exact(a.c.tail_k + bh * kGroup * D, tail_count, 0, SPLIT ? 32 * NW : 64 * NW);
    else if (pres)
      stage_k_record();
  };
  auto stage_v_tile = [&](int u, bool pres) {
    if (has_tail && u == T - 1)
      stage_v_exact(a.c.tail_v + bh * kGroup * D, tail_count, SPLIT ? 32 * NW : 0, SPLIT ? 32 * NW : 64 * NW);
    else if (pres)
      stage_v_record();
  };

  bool present = true;   // tile t has storage
  if constexpr (SPLIT) {
    // Eight-wave workgroups, one loop per wave half (so that the query
    // operand the V-staging waves hold across their V staging is not kept
    // live through the K-staging waves' steps).  Per tile, between barrier B
    // and barrier A the V-staging waves stage the tile's V half, so they
    // form the next tile's query operand after their PV instead, where they
    // would otherwise wait for the K staging; that needs the next record's
    // c^K in LDS before barrier A, so wave 1 stages it at the end of its
    // softmax, into the other of the two c^K buffers.
    if (!vrole) {
#pragma unroll 1
      for (int t = 0; t < T; ++t) {
        // Per-lane index math of the staging and masking (tens of values) is
        // cheaper to recompute per tile than to keep live across the loop.
        asm volatile("" : "+v"(tid));
        l = tid & 63;
        const bool exact = t == 0 || (has_tail && t == T - 1);
        const int base = t == 0 ? 0 : exact ? tail_base : kSink + kGroup * (t - 1);
        const int count = !present ? 0 : t == 0 ? min(nseq, kSink) : exact ? tail_count : kGroup;
        if (exact) {
          load_exact_query();
          f = qk_scale;
        }
        const bool np = issue_next(t);
        phase_end(pc, 0);   // next record's loads issued
        if (!exact) f = record_operand(t & 1);
        phase_end(pc, 1);
        qk_products();
        phase_end(pc, 2);
        softmax(base, count);
        if (role == 1 && np && t + 1 <= n_rec) stage_ck((t + 1) & 1);
        phase_end(pc, 3);
        if (t + 1 < T) {
          lds_barrier();   // every wave is done with this K tile
          phase_end(pc, 4);
          stage_k_tile(t + 1, np);
        }
        phase_end(pc, 5);
        pv(exact);
        phase_end(pc, 6);
        if (t + 1 < T) lds_barrier();   // every wave is done with this V tile
        phase_end(pc, 7);
        present = np;
      }
    } else {
      load_exact_query();   // tile 0, the sink
      f = qk_scale;
#pragma unroll 1
      for (int t = 0; t < T; ++t) {
        asm volatile("" : "+v"(tid));   // as above
        l = tid & 63;
        const bool exact = t == 0 || (has_tail && t == T - 1);
        const int base = t == 0 ? 0 : exact ? tail_base : kSink + kGroup * (t - 1);
        const int count = !present ? 0 : t == 0 ? min(nseq, kSink) : exact ? tail_count : kGroup;
        const bool np = issue_next(t);
        phase_end(pc, 0);
        qk_products();   // operand formed in the previous tile's last window
        phase_end(pc, 2);
        softmax(base, count);
        phase_end(pc, 3);
        if (t + 1 < T) lds_barrier();
        phase_end(pc, 4);
        pv(exact);
        phase_end(pc, 6);
        if (t + 1 < T) {
          // the next tile's query operand (its c^K was staged before barrier A;
          // no record loads are in flight for a next tile that is the tail)
          if (has_tail && t + 1 == T - 1) {
            load_exact_query();
            f = qk_scale;
          } else {
            f = record_operand((t + 1) & 1);
          }
          phase_end(pc, 1);
          lds_barrier();
          phase_end(pc, 7);
          stage_v_tile(t + 1, np);
        }
        phase_end(pc, 8);
        present = np;
      }
    }
  } else {
#pragma unroll 1
    for (int t = 0; t < T; ++t) {
      asm volatile("" : "+v"(tid));   // as above
      l = tid & 63;
      const bool exact = t == 0 || (has_tail && t == T - 1);
      const int base = t == 0 ? 0 : exact ? tail_base : kSink + kGroup * (t - 1);
      const int count = !present ? 0 : t == 0 ? min(nseq, kSink) : exact ? tail_count : kGroup;
      if (exact) {
        load_exact_query();
        f = qk_scale;
      }
      const bool np = issue_next(t);
      phase_end(pc, 0);   // next record's loads issued
      if (!exact) f = record_operand(0);
      phase_end(pc, 1);
      qk_products();
      phase_end(pc, 2);
      softmax(base, count);
      phase_end(pc, 3);
      // the next tile's K half, once every wave is done with this K tile
      if (t + 1 < T) {
        lds_barrier();
        phase_end(pc, 4);
        stage_k_tile(t + 1, np);
      }
      phase_end(pc, 5);
      pv(exact);
      phase_end(pc, 6);
      // the next tile's V half, once every wave is done with this V tile
      if (t + 1 < T) {
        lds_barrier();
        phase_end(pc, 7);
        stage_v_tile(t + 1, np);
      }
      phase_end(pc, 8);
      present = np;
    }
  }
  phase_store(((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * NW + w, pc);

  if (rotated) rotate_out<NCT>(o, G);
  if (prow >= 0) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* out = a.out + (((int64_t)b * C + blockIdx.x * POS + r_lane / GQ) * a.hq + kvh * GQ + r_lane % GQ) * D;
#pragma unroll
    for (int c = 0; c < NCT; ++c) *reinterpret_cast<v4f*>(out + 16 * c + 4 * G) = o[c] * inv;
  }
}

#ifdef KVARN_WAVE_TRACE
hipError_t trace_io_prefill_attn(void* host, size_t bytes) { return trace_io_local(host, bytes); }
#endif

template <int D, int MAXB, int NW>
static void launch_pa_w(int gq, const PrefillAttnArgs& a, hipStream_t st) {
  const int pos = 16 * NW / gq;
  const dim3 grid((a.chunk + pos - 1) / pos, a.c.hkv, a.c.batch);
  if (gq == 1)
    hipLaunchKernelGGL((prefill_attn_kernel<D, 1, MAXB, NW>), grid, dim3(64 * NW), 0, st, a);
  else if (gq == 2)
    hipLaunchKernelGGL((prefill_attn_kernel<D, 2, MAXB, NW>), grid, dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<D, 4, MAXB, NW>), grid, dim3(64 * NW), 0, st, a);
}

// Eight-wave workgroups at D 128 when their grid has at least one per CU
// (2,048-token chunk at the Llama-3.1-8B shape: 2.81 -> 2.42 ms); a shorter
// chunk keeps four-wave workgroups, which spread over twice as many CUs
// (512 tokens: 1.14 ms, against 1.22 ms with eight-wave workgroups).
template <int D, int MAXB>
static void launch_pa_d(int gq, const PrefillAttnArgs& a, hipStream_t st) {
  if constexpr (D == 128) {
    const int64_t wgs8 = (int64_t)((a.chunk * gq + 127) / 128) * a.c.hkv * a.c.batch;
    const int cus = decode_cu_count();
    if (cus > 0 && wgs8 >= cus) {
      launch_pa_w<D, MAXB, 8>(gq, a, st);
      return;
    }
  }
  launch_pa_w<D, MAXB, 4>(gq, a, st);
}

hipError_t launch_prefill_attn(int D, int gq, const PrefillAttnArgs& a, hipStream_t st) {
  if (a.chunk <= 0) return hipSuccess;
  const bool wide = a.k_bits > 4 || a.v_bits > 4;
  if (D == 128) {
    if (wide)
      launch_pa_d<128, 8>(gq, a, st);
    else
      launch_pa_d<128, 4>(gq, a, st);
  } else {
    if (wide)
      launch_pa_d<256, 8>(gq, a, st);
    else
      launch_pa_d<256, 4>(gq, a, st);
  }
  return hipGetLastError();
}

}  // namespace kvarn
