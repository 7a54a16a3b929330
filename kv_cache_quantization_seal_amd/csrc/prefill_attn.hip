// KVarN chunked-prefill attention on gfx950: the queries of a prefill chunk
// (the last C cached positions of each request) attend causally over the
// cache as it holds them -- the exact fp16 sink and tail, and the sealed
// groups read directly from their records -- on fp16 MFMA with fp32
// accumulation ["KVarN KV Cache: Implementation and Benchmarks"
// (anbeeld.com), §2.1 "Sink, Body, And Tail": attention paths read the
// records; §1 "Where KVarN Comes From": attention runs in the rotated frame
// and the output is rotated back once].
//
// Workgroup = 4 waves = 64 query rows of one (request, KV head): row
// r = position-in-tile * GQ + head, so the GQ query heads of a KV head share
// every key tile staged in LDS.  Each wave owns 16 rows (the MFMA M).  The
// workgroup walks the key tiles of its request in position order -- sink,
// records, tail, each 128 tokens at most, up to its last row's position --
// with an online softmax per row, all in the rotated frame:
//   * record tile: the codes minus the mid level, exact in fp16, are staged
//     as the B operand; the query operand is q~ = q_r * c^K (fp32, split into
//     fp16 hi + lo, two MFMAs); logit = s^K_t * (q~ . (code - mid));
//     PV: w = p * s^V_t (hi + lo) against V codes - mid, then times c^V_j;
//   * exact tile (sink, tail): the fp16 rows are rotated in fp32 and staged
//     as hi + lo fp16 pairs (three MFMAs: hi*hi, hi*lo, lo*hi), scales 1.
// Every fp32 operand split into hi + lo is first scaled, per row, by the power
// of two that puts the row's largest magnitude in [2^11, 2^12): its low parts
// then stay fp16 normals (a subnormal low part would leave only the 11 bits
// of the high part); the scale is undone exactly on the fp32 results.
// One inverse Hadamard per row at the end, across the output accumulators.
//
// MFMA v_mfma_f32_16x16x32_f16 lane layout (checked on the device): A lane l
// holds row l%16, k = 8(l/16)..+7; B lane l holds column l%16, same k; C lane
// l holds column l%16, rows 4(l/16)..+3.
#include "common.hpp"
#include "kernels.hpp"

namespace kvarn {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
constexpr int kPaWaves = 4;
constexpr int kPaRows = 16;  // rows per wave
constexpr float kPaLog2e = 1.4426950408889634f;

template <int D>
struct PaSmem {
  static constexpr int KP = D + 8;    // pitch of a K tile row (token), halves
  static constexpr int VP = 128 + 8;  // pitch of a V tile row (channel), halves
  static constexpr int TILE = 128 * KP > D * VP ? 128 * KP : D * VP;
  alignas(16) _Float16 hi[TILE];
  alignas(16) _Float16 lo[TILE];      // exact tiles only
  float sk[128], sv[128];              // token scales of the tile (1 for exact tiles)
  float ck[D], cv[D];                  // channel scales (1 for exact tiles)
  alignas(16) _Float16 p[kPaWaves][2][kPaRows][32 + 8];  // w hi / lo of one 32-token step
  float qscale[kPaWaves][kPaRows];   // per-row inverse scale of the query operand
};

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

// Exact tile: `count` fp16 rows [128][D] at src (rows past count are zero),
// rotated, as hi + lo fp16 into the K layout [token][KP] (TRANSPOSE false) or
// the V layout [channel][VP] (TRANSPOSE true).  All threads.
template <int D, bool TRANSPOSE>
__device__ void stage_exact(PaSmem<D>& sm, const __half* __restrict__ src, int count, int tid) {
  constexpr int NT = D / 64, TPP = 256 / NT;
#pragma unroll 1
  for (int pass = 0; pass < 128 / TPP; ++pass) {
    const int t = pass * TPP + tid / NT, chunk = tid % NT;
    float x[64];
    load64h(x, src + (size_t)t * D + 64 * chunk, t < count);
    rotate64<D>(x, chunk);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const _Float16 h = (_Float16)x[i];
      const _Float16 l = (_Float16)(x[i] - (float)h);
      const int j = 64 * chunk + i;
      const int idx = TRANSPOSE ? j * PaSmem<D>::VP + t : t * PaSmem<D>::KP + j;
      sm.hi[idx] = h;
      sm.lo[idx] = l;
    }
  }
}

// 64 codes of BITS bits (a little-endian bit stream starting at bit 0 of
// w[0]) minus the mid level, as fp16 (exact: half-integers below 2^8).
template <int BITS>
__device__ __forceinline__ void codes64(const uint8_t* __restrict__ src, _Float16* __restrict__ dst) {
  constexpr int NW = 2 * BITS;  // 64 * BITS / 32 dwords
  constexpr float MID = 0.5f * ((1 << BITS) - 1);
  uint32_t w[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) w[k] = reinterpret_cast<const uint32_t*>(src)[k];
  v8h out[8];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const int bit = BITS * i, wi = bit >> 5, sh = bit & 31;
    uint32_t v;
    if (sh + BITS <= 32)
      v = (w[wi] >> sh) & ((1u << BITS) - 1);
    else
      v = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << BITS) - 1);
    out[i >> 3][i & 7] = (_Float16)((float)v - MID);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) reinterpret_cast<v8h*>(dst)[k] = out[k];
}

// Record tile: the codes of one record (kind K: rows = 128 tokens of D codes,
// into [token][KP]; kind V: rows = D channels of 128 codes, into
// [channel][VP]) as fp16 code - mid.  All threads.
template <int D, bool VKIND>
__device__ void stage_codes(PaSmem<D>& sm, const uint8_t* __restrict__ rec, int bits, int tid) {
  constexpr int ROWS = VKIND ? D : 128, CODES = VKIND ? 128 : D, PITCH = VKIND ? PaSmem<D>::VP : PaSmem<D>::KP;
  constexpr int ITEMS = ROWS * CODES / 64;
#pragma unroll 1
  for (int it = tid; it < ITEMS; it += 256) {
    const int r = it / (CODES / 64), ch = it % (CODES / 64);
    const uint8_t* src = rec + (size_t)r * (CODES * bits / 8) + ch * 8 * bits;
    _Float16* dst = sm.hi + r * PITCH + 64 * ch;
    switch (bits) {
      case 2: codes64<2>(src, dst); break;
      case 3: codes64<3>(src, dst); break;
      case 4: codes64<4>(src, dst); break;
      case 5: codes64<5>(src, dst); break;
      case 6: codes64<6>(src, dst); break;
      default: codes64<8>(src, dst); break;
    }
  }
}

__device__ __forceinline__ v8h ld8(const _Float16* p) { return *reinterpret_cast<const v8h*>(p); }

}  // namespace

template <int D, int GQ>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillAttnArgs a) {
  __shared__ PaSmem<D> sm;
  constexpr int KS = D / 32;   // MFMA k-steps over the channels
  constexpr int NCT = D / 16;  // output channel tiles
  constexpr int POS = 64 / GQ; // positions per workgroup
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int G = l >> 4, n = l & 15;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int nseq = a.c.seq_len[b];
  const int C = a.chunk;
  const int64_t bh = (int64_t)b * a.c.hkv + kvh;
  // Position of workgroup row r (or -1 if the row is outside the chunk).
  auto row_pos = [&](int r) {
    const int i = blockIdx.x * POS + r / GQ;
    const int p = nseq - C + i;
    return (i < C && p >= 0) ? p : -1;
  };
  int pmax = -1;
#pragma unroll 1
  for (int r = 0; r < 64; ++r) pmax = max(pmax, row_pos(r));

  // ---- queries: rotated and scaled by softmax_scale * log2(e), staged in
  // LDS (fp32, 64 rows x D) through the K tile space, then read in A order.
  {
    float* qs = reinterpret_cast<float*>(sm.hi);   // 64 x D fp32 fits in the tile space
    constexpr int NT = D / 64;
#pragma unroll 1
    for (int it = tid; it < 64 * NT; it += 256) {
      const int r = it / NT, chunk = it % NT;
      const int p = row_pos(r);
      const int hq = kvh * GQ + r % GQ;
      const int i = blockIdx.x * POS + r / GQ;
      float x[64];
      load64h(x, a.q + (((int64_t)b * C + (p >= 0 ? i : 0)) * a.hq + hq) * D + 64 * chunk, p >= 0);
      // rotate64 needs the NT threads of a row in adjacent lanes: it = r*NT + chunk
      rotate64<D>(x, chunk);
#pragma unroll
      for (int k = 0; k < 64; ++k) qs[r * D + 64 * chunk + k] = x[k] * a.scale * kPaLog2e;
    }
  }
  lds_barrier();
  float qr[KS][8];   // A operand order: row 16w + n', n' = l % 16; channels 32s + 8G + e
  {
    const float* qs = reinterpret_cast<const float*>(sm.hi);
    const int r = 16 * w + n;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[s][e] = qs[r * D + 32 * s + 8 * G + e];
  }
  // C-layout rows of this lane: 16w + 4G + i.
  int prow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) prow[i] = row_pos(16 * w + 4 * G + i);

  float m_run[4], l_run[4];
  v4f o[NCT];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c) o[c] = v4f{0.f, 0.f, 0.f, 0.f};

  const int n_groups = nseq > kSink ? min((nseq - kSink) / kGroup, a.c.max_groups) : 0;
  const int n_tiles = 1 + n_groups + 1;   // sink, records, tail
#pragma unroll 1
  for (int tile = 0; tile < n_tiles; ++tile) {
    // Tile positions [base, base + count) and its storage.
    int base, count;
    const uint8_t* rec = nullptr;
    const bool exact = tile == 0 || tile == n_tiles - 1;
    if (tile == 0) {
      base = 0;
      count = min(nseq, kSink);
    } else if (tile == n_tiles - 1) {
      base = kSink + kGroup * n_groups;
      count = nseq > base ? nseq - base : 0;
    } else {
      base = kSink + kGroup * (tile - 1);
      count = kGroup;
      const int64_t off = pair_offset(a.c.map, b, kvh, tile - 1, a.c.hkv, a.c.max_groups, a.c.group_bytes);
      if (off < 0) continue;   // no storage: the group is absent (uniform over the workgroup)
      rec = a.c.records + off;
    }
    if (count <= 0 || base > pmax) continue;   // uniform over the workgroup

    lds_barrier();   // the previous tile's V operands have been read
    // ---- stage K and every scale of the tile
    if (exact) {
      const __half* src = (tile == 0 ? a.c.sink_k : a.c.tail_k) + bh * kGroup * D;
      stage_exact<D, false>(sm, src, count, tid);
      for (int t = tid; t < 128; t += 256) sm.sk[t] = sm.sv[t] = 1.f;
      for (int j = tid; j < D; j += 256) sm.ck[j] = sm.cv[j] = 1.f;
    } else {
      stage_codes<D, false>(sm, rec, a.k_bits, tid);
      const int kcode = kGroup * D * a.k_bits / 8, vrec = a.c.rec_k_bytes, vcode = kGroup * D * a.v_bits / 8;
      const uint16_t* sK = reinterpret_cast<const uint16_t*>(rec + kcode);
      const uint16_t* sV = reinterpret_cast<const uint16_t*>(rec + vrec + vcode);
      for (int t = tid; t < 128; t += 256) {
        sm.sk[t] = h2f(sK[t]);
        sm.sv[t] = h2f(sV[t]);
      }
      for (int j = tid; j < D; j += 256) {
        sm.ck[j] = h2f(sK[kGroup + j]);
        sm.cv[j] = h2f(sV[kGroup + j]);
      }
    }
    lds_barrier();

    // ---- QK: logits of the wave's 16 rows x 128 tokens (8 token tiles).
    // q~ of row n, scaled by a power of two per row (its inverse goes to the
    // C-layout lanes of that row through the wave's LDS area).
    v8h ahi[KS], alo[KS];
    {
      float qt[KS][8];
      float mx = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qt[s][e] = qr[s][e] * sm.ck[32 * s + 8 * G + e];
          mx = fmaxf(mx, fabsf(qt[s][e]));
        }
      float inv;
      const float sc = pow2_scale(max_over_groups(mx), inv);
      if (G == 0) sm.qscale[w][n] = inv;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = qt[s][e] * sc;
          const _Float16 h = (_Float16)x;
          ahi[s][e] = h;
          alo[s][e] = (_Float16)(x - (float)h);
        }
    }
    wave_sync();
    float qinv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qinv[i] = sm.qscale[w][4 * G + i];
    float lg[8][4];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const _Float16* krow = sm.hi + (16 * tt + n) * PaSmem<D>::KP + 8 * G;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const v8h bk = ld8(krow + 32 * s);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s], bk, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[s], bk, acc, 0, 0, 0);
      }
      if (exact) {
        const _Float16* klo = sm.lo + (16 * tt + n) * PaSmem<D>::KP + 8 * G;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s], ld8(klo + 32 * s), acc, 0, 0, 0);
      }
      const int tok = 16 * tt + n;
      const float st = sm.sk[tok];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lg[tt][i] = (tok < count && base + tok <= prow[i]) ? acc[i] * (st * qinv[i]) : -INFINITY;
    }

    // ---- online softmax per row (row 4G + i of the wave spans the 16 lanes of DPP row G)
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = lg[0][i];
#pragma unroll
      for (int tt = 1; tt < 8; ++tt) mx = fmaxf(mx, lg[tt][i]);
      mx = row16_max(mx);
      const float m_new = fmaxf(m_run[i], mx);
      alpha[i] = (m_new == -INFINITY || m_run[i] == -INFINITY) ? (m_new == -INFINITY ? 1.f : 0.f)
                                                                 : __builtin_amdgcn_exp2f(m_run[i] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const float p = lg[tt][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lg[tt][i] - m_new);
        ps += p;
        lg[tt][i] = p * sm.sv[16 * tt + n];   // w = p * s^V (1 for exact tiles)
      }
      l_run[i] = fmaf(l_run[i], alpha[i], row16_sum(ps));
      m_run[i] = m_new;
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[c][i] *= alpha[i];

    // ---- w as the PV A operand (hi + lo), scaled per row by a power of two,
    // through the wave's LDS area: token step u = token tiles 2u, 2u + 1
    float winv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = 0.f;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) mx = fmaxf(mx, lg[tt][i]);
      const float sc = pow2_scale(row16_max(mx), winv[i]);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) lg[tt][i] *= sc;
    }
    v8h whi[4], wlo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = lg[2 * u + q][i];
          const _Float16 h = (_Float16)x;
          sm.p[w][0][4 * G + i][16 * q + n] = h;
          sm.p[w][1][4 * G + i][16 * q + n] = (_Float16)(x - (float)h);
        }
      }
      wave_sync();
      whi[u] = ld8(&sm.p[w][0][n][8 * G]);
      wlo[u] = ld8(&sm.p[w][1][n][8 * G]);
      wave_sync();
    }

    lds_barrier();   // every wave is done with the K tile
    // ---- stage V
    if (exact)
      stage_exact<D, true>(sm, (tile == 0 ? a.c.sink_v : a.c.tail_v) + bh * kGroup * D, count, tid);
    else
      stage_codes<D, true>(sm, rec + a.c.rec_k_bytes, a.v_bits, tid);
    lds_barrier();

    // ---- PV: channel tiles of 16, token steps of 32; records scale by c^V
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      const _Float16* vrow = sm.hi + (16 * ct + n) * PaSmem<D>::VP + 8 * G;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v8h bv = ld8(vrow + 32 * u);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(whi[u], bv, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wlo[u], bv, acc, 0, 0, 0);
      }
      if (exact) {
        const _Float16* vlo = sm.lo + (16 * ct + n) * PaSmem<D>::VP + 8 * G;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(whi[u], ld8(vlo + 32 * u), acc, 0, 0, 0);
      }
      const float cvj = sm.cv[16 * ct + n];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[ct][i] = fmaf(cvj * winv[i], acc[i], o[ct][i]);
    }
  }

  // ---- normalize, rotate back (H symmetric: channel 16 ct + n; butterflies
  // over the bits of ct in registers, over the bits of n across the row's
  // lanes), write the rows of this lane.
#pragma unroll
  for (int st = 1; st < NCT; st <<= 1) {
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      if (!(c & st)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u = o[c][i], v = o[c + st][i];
          o[c][i] = u + v;
          o[c + st][i] = u - v;
        }
      }
    }
  }
#pragma unroll
  for (int st = 1; st < 16; st <<= 1) {
    const bool upper = n & st;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = dpp_pair_f(o[c][i], st);
        o[c][i] = upper ? pv - o[c][i] : o[c][i] + pv;
      }
  }
  const float rs = D == 128 ? 0.08838834764831845f : 0.0625f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * G + i;
    if (prow[i] < 0) continue;
    const int pi = blockIdx.x * POS + r / GQ;
    const int hq = kvh * GQ + r % GQ;
    const float inv = l_run[i] > 0.f ? rs / l_run[i] : 0.f;
    float* out = a.out + (((int64_t)b * C + pi) * a.hq + hq) * D;
#pragma unroll
    for (int c = 0; c < NCT; ++c) out[16 * c + n] = o[c][i] * inv;
  }
}

template <int D>
static void launch_pa_d(int gq, const PrefillAttnArgs& a, hipStream_t st) {
  const int pos = 64 / gq;
  const dim3 grid((a.chunk + pos - 1) / pos, a.c.hkv, a.c.batch);
  if (gq == 1)
    hipLaunchKernelGGL((prefill_attn_kernel<D, 1>), grid, dim3(256), 0, st, a);
  else if (gq == 2)
    hipLaunchKernelGGL((prefill_attn_kernel<D, 2>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<D, 4>), grid, dim3(256), 0, st, a);
}

hipError_t launch_prefill_attn(int D, int gq, const PrefillAttnArgs& a, hipStream_t st) {
  if (a.chunk <= 0) return hipSuccess;
  if (D == 128)
    launch_pa_d<128>(gq, a, st);
  else
    launch_pa_d<256>(gq, a, st);
  return hipGetLastError();
}

}  // namespace kvarn
