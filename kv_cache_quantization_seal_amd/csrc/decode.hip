// KVarN decode attention on gfx950: split-K over sealed groups, exact sink and
// tail, one inverse rotation per query head.
//
// The query is rotated by the same Hadamard matrix as the stored K and V, so
// q.k is unchanged and attention over the records runs in the rotated frame;
// the record part of the output is rotated back once per query head
// ["KVarN KV Cache: Implementation and Benchmarks" (anbeeld.com), §1 "Where
// KVarN Comes From"].  Sink and tail are exact fp16 and are read in the
// original frame; records are read directly, never expanded in memory (same
// page, §2.1 "Sink, Body, And Tail").
//
// Record splits.  A workgroup (4 waves) walks a range of 128-token groups of
// one (request, KV head).  Each group's K and V records are copied into a
// double-buffered LDS slot (the next group's loads are in flight while the
// current one is computed) and the four waves share the work:
//   logit_t = s^K_t * sum_j q~_j (code_tj - mid),  q~ = q_r * c^K * scale,
//   w_t = p_t * s^V_t,  o_rot_j += c^V_j * sum_t w_t (code_tj - mid).
// Both sums run on v_mfma_i32_16x16x64_i8 with the codes as exact int8
// operands.  q~ and w are split into three radix-128 int8 limbs
// x * inv ~ a0 + a1/128 + a2/128^2 (|error| <= 0.5/128^2 of the group maximum
// scaled to the top-limb range); the 16 MFMA rows carry (head, limb) pairs,
// so each lane holds every limb of one head and recombines them exactly in
// int32, with one conversion to fp32.
//   wave h < GQ : q~ limbs of head h;
//   wave w      : QK for token tiles nt = 2w, 2w+1; PV for channel tiles
//                 ct = w*(D/64) .. w*(D/64) + D/64 - 1.
// Softmax maxima per head are exchanged through LDS (base-2 online softmax).
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
#include "common.hpp"
#include "kernels.hpp"

namespace kvarn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kExactTok = 16;  // exact tokens per wave per round

typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int D, int KB, int VB>
struct RecGeom {
  static constexpr int KS = D / 64;                      // QK K-steps
  static constexpr int NCT = D / 16;                     // PV channel tiles
  static constexpr int CTW = NCT / kWaves;               // channel tiles per wave
  static constexpr int LBK = KS * 2 * KB;                // K-code bytes per lane per token
  static constexpr int LBV = 4 * VB;                     // V-code bytes per lane per channel
  static constexpr int KROW = D * KB / 8;                // bytes of one token row of K codes
  static constexpr int VROW = kGroup * VB / 8;           // bytes of one channel row of V codes
  static constexpr int KCODE = kGroup * D * KB / 8;
  static constexpr int VCODE = kGroup * D * VB / 8;
  static constexpr int KREC = KCODE + 2 * kGroup + 2 * D;
  static constexpr int VREC = VCODE + 2 * kGroup + 2 * D;
  static constexpr int GB = KREC + VREC;                 // staged bytes per group
  static constexpr int CHUNKS = GB / 16;
  static constexpr int CPT = (CHUNKS + 255) / 256;       // 16-byte chunks per thread
};

template <int D, int KB, int VB, int GQ>
struct alignas(16) RecSmem {
  alignas(16) uint8_t buf[2][RecGeom<D, KB, VB>::GB];  // staged K record | V record
  alignas(16) uint8_t ql[GQ][3][D];                    // q~ limbs, operand order
  alignas(16) uint8_t wl[GQ][3][kGroup];               // w limbs, operand order
  float qx[GQ][D];                                     // scaled query, rotated in place
  float e[GQ];                                         // q~ maximum per head (this group)
  float pmax[kWaves][GQ];                              // per-wave partial maxima
  float lsum[kWaves][GQ];
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

template <int VB>
__device__ __forceinline__ int tok_of(int nt, int n) {
  return 16 * (n >> 1) + unpack_index<VB>(8 * (n & 1) + nt);
}

// Buffer resource over `bytes` bytes at a wave-uniform base; loads past the
// end return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Largest |top limb| so that sum_j A_j (2 code_j - L) fits int32, with
// A_j = a0*2^14 + a1*2^7 + a2 and |a1|,|a2| <= 64, over k_terms terms.
__host__ __device__ constexpr float top_limb(int k_terms, int levels) {
  return (k_terms * levels <= 768) ? 127.0f : (k_terms * levels <= 1920 ? 63.0f : 31.0f);
}

__device__ __forceinline__ void store_partial_ml(const DecodeArgs& a, int b, int hq_idx, int split, float m, float l) {
  const int64_t row = ((int64_t)b * a.hq + hq_idx) * a.nsplit + split;
  a.ws_ml[2 * row] = m;
  a.ws_ml[2 * row + 1] = l;
}

// ---------------------------------------------------------------------------
// Record split (workgroup-cooperative)
// ---------------------------------------------------------------------------
template <int D, int KB, int VB, int GQ>
__device__ void record_split(RecSmem<D, KB, VB, GQ>& sm, const DecodeArgs& a, int b, int kvh, int split,
                             int nseq) {
  using Gm = RecGeom<D, KB, VB>;
  constexpr int KS = Gm::KS, CTW = Gm::CTW, CPT = Gm::CPT;
  constexpr int LK = (1 << KB) - 1, LV = (1 << VB) - 1;
  constexpr float QMAX = top_limb(D, LK);
  constexpr float WMAX = top_limb(kGroup, LV);
  constexpr int QPL = D / 64;  // q~ values produced per lane (wave h < GQ)
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int G = l >> 4, n = l & 15;
  const bool hvalid = G < GQ;
  const int hm = n >> 2, im = n & 3;  // A-operand row of this lane: (head, limb)
  const bool arow_valid = hm < GQ && im < 3;

  const uint8_t* recs = a.c.records + (((int64_t)b * a.c.hkv + kvh) * a.c.max_groups) * a.c.group_bytes;
  const int g0 = split * a.groups_per_split;
  const int gcap = min(g0 + a.groups_per_split, a.c.max_groups);  // slots that exist
  const int n_groups = nseq > kSink ? min((nseq - kSink) / kGroup, a.c.max_groups) : 0;
  const int g1 = min(gcap, n_groups);

  // The first group's stage loads go out before anything else (the slot
  // exists, so the load is safe before seq_len decides whether it is used).
  v4u stage[CPT];
  auto load_stage = [&](int g) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(recs + (int64_t)g * a.c.group_bytes, Gm::GB);
#pragma unroll
    for (int k = 0; k < CPT; ++k) stage[k] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (tid + 256 * k), 0, 0);
  };
  auto store_stage = [&](uint8_t* dst) {
#pragma unroll
    for (int k = 0; k < CPT; ++k)
      if (tid + 256 * k < Gm::CHUNKS) *reinterpret_cast<v4u*>(dst + 16 * (tid + 256 * k)) = stage[k];
  };
  if (g0 < gcap) load_stage(g0);

  // Scaled query (log2 domain) of the GQ heads, rotated: qx <- qx H_D.
  for (int idx = tid; idx < GQ * D; idx += 256) {
    const int h = idx / D, j = idx % D;
    sm.qx[h][j] = __half2float(a.q[((int64_t)b * a.hq + kvh * GQ + h) * D + j]) * a.scale * kLog2e;
  }
  __syncthreads();
  for (int s = 1; s < D; s <<= 1) {
    for (int idx = tid; idx < GQ * D / 2; idx += 256) {
      const int h = idx / (D / 2), rr = idx % (D / 2);
      const int lo = ((rr & ~(s - 1)) << 1) | (rr & (s - 1));
      const float x0 = sm.qx[h][lo], x1 = sm.qx[h][lo + s];
      sm.qx[h][lo] = x0 + x1;
      sm.qx[h][lo + s] = x0 - x1;
    }
    __syncthreads();
  }
  // q~ producer (wave w < GQ, head w): operand bytes [QPL*l, QPL*l + QPL).
  const float rs = (D == 128) ? 0.08838834764831845f : 0.0625f;
  float qr[QPL];
  int qch[QPL];
#pragma unroll
  for (int e = 0; e < QPL; ++e) {
    const int ob = QPL * l + e;
    qch[e] = 16 * (ob >> 4) + unpack_index<KB>(ob & 15);
    qr[e] = w < GQ ? sm.qx[w][qch[e]] * rs : 0.f;
  }
  if (g0 < g1) store_stage(sm.buf[0]);
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;  // head G (replicated in every wave)
  float o_acc[CTW];
#pragma unroll
  for (int c = 0; c < CTW; ++c) o_acc[c] = 0.f;

  for (int g = g0, it = 0; g < g1; ++g, ++it) {
    const uint8_t* cur = sm.buf[it & 1];
    const bool more = g + 1 < g1;
    if (more) load_stage(g + 1);
    const uint16_t* sk16 = reinterpret_cast<const uint16_t*>(cur + Gm::KCODE);
    const uint16_t* ck16 = sk16 + kGroup;
    const uint16_t* sv16 = reinterpret_cast<const uint16_t*>(cur + Gm::KREC + Gm::VCODE);
    const uint16_t* cv16 = sv16 + kGroup;

    // (A) q~ limbs of head w.
    if (w < GQ) {
      float y[QPL];
      float ym = 0.f;
#pragma unroll
      for (int e = 0; e < QPL; ++e) {
        y[e] = qr[e] * h2f(ck16[qch[e]]);
        ym = fmaxf(ym, fabsf(y[e]));
      }
      const float E = wave_max(ym);
      const float inv = E > 0.f ? QMAX * __builtin_amdgcn_rcpf(E) : 0.f;
      float f0[QPL], f1[QPL], f2[QPL];
#pragma unroll
      for (int e = 0; e < QPL; ++e) limbs_r128(y[e], inv, f0[e], f1[e], f2[e]);
      uint8_t* base = &sm.ql[w][0][QPL * l];
      if constexpr (QPL == 2) {
        const uint32_t b0 = __builtin_amdgcn_perm(__float_as_uint(f0[1]), __float_as_uint(f0[0]), 0x0c0c0400u);
        const uint32_t b1 = __builtin_amdgcn_perm(__float_as_uint(f1[1]), __float_as_uint(f1[0]), 0x0c0c0400u);
        const uint32_t b2 = __builtin_amdgcn_perm(__float_as_uint(f2[1]), __float_as_uint(f2[0]), 0x0c0c0400u);
        *reinterpret_cast<uint16_t*>(base) = (uint16_t)b0;
        *reinterpret_cast<uint16_t*>(base + D) = (uint16_t)b1;
        *reinterpret_cast<uint16_t*>(base + 2 * D) = (uint16_t)b2;
      } else {
        *reinterpret_cast<uint32_t*>(base) = pack_low_bytes(f0[0], f0[1], f0[2], f0[3]);
        *reinterpret_cast<uint32_t*>(base + D) = pack_low_bytes(f1[0], f1[1], f1[2], f1[3]);
        *reinterpret_cast<uint32_t*>(base + 2 * D) = pack_low_bytes(f2[0], f2[1], f2[2], f2[3]);
      }
      if (l == 0) sm.e[w] = E;
    }
    __syncthreads();  // B1: q~ limbs ready

    // (B) QK for token tiles 2w, 2w+1.
    v4i aq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (arow_valid) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sm.ql[hm][im][16 * (G * KS + s)]);
        aq[s] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {
        aq[s] = v4i{0, 0, 0, 0};
      }
    }
    v4i sacc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) sacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[s], ones, sacc, 0, 0, 0);
    const uint32_t negls =
        0u - (uint32_t)LK * (((uint32_t)sacc[0] << 14) + ((uint32_t)sacc[1] << 7) + (uint32_t)sacc[2]);
    const float kscale = (hvalid ? sm.e[G] : 0.f) * (1.0f / (QMAX * 32768.0f));
    float logit[2];
    float lmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int nt = 2 * w + t;
      const int tok = tok_of<VB>(nt, n);
      const uint8_t* kp = cur + tok * Gm::KROW + G * Gm::LBK;
      uint32_t kw[Gm::LBK / 4];
#pragma unroll
      for (int k = 0; k < Gm::LBK / 4; ++k) kw[k] = reinterpret_cast<const uint32_t*>(kp)[k];
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[s], unpack16<KB>(&kw[s * (KB / 2)]), acc, 0, 0, 0);
      const uint32_t x = ((uint32_t)acc[0] << 14) + ((uint32_t)acc[1] << 7) + (uint32_t)acc[2];
      const int yv = (int)((x << 1) + negls);
      logit[t] = hvalid ? (float)yv * (h2f(sk16[tok]) * kscale) : -INFINITY;
      lmax = fmaxf(lmax, logit[t]);
    }
    lmax = row16_max(lmax);
    if (n == 0 && hvalid) sm.pmax[w][G] = lmax;
    __syncthreads();  // B2: logit maxima
    float gmax = -INFINITY;
    if (hvalid) {
#pragma unroll
      for (int k = 0; k < kWaves; ++k) gmax = fmaxf(gmax, sm.pmax[k][G]);
    }
    const float m_new = fmaxf(m_run, gmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float wv[2];
    float psum = 0.f, wmax = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float p = hvalid ? __builtin_amdgcn_exp2f(logit[t] - m_new) : 0.f;
      psum += p;
      wv[t] = p * h2f(sv16[tok_of<VB>(2 * w + t, n)]);
      wmax = fmaxf(wmax, wv[t]);
    }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int c = 0; c < CTW; ++c) o_acc[c] *= alpha;
    wmax = row16_max(wmax);
    __syncthreads();  // everyone has read pmax (reused below)
    if (n == 0 && hvalid) sm.pmax[w][G] = wmax;
    __syncthreads();  // B3: w maxima
    float W = 0.f;
    if (hvalid) {
#pragma unroll
      for (int k = 0; k < kWaves; ++k) W = fmaxf(W, sm.pmax[k][G]);
    }
    const float winv = W > 0.f ? WMAX * __builtin_amdgcn_rcpf(W) : 0.f;
    if (hvalid) {
      float f0[2], f1[2], f2[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) limbs_r128(wv[t], winv, f0[t], f1[t], f2[t]);
      uint8_t* base = &sm.wl[G][0][8 * n + 2 * w];
      *reinterpret_cast<uint16_t*>(base) =
          (uint16_t)__builtin_amdgcn_perm(__float_as_uint(f0[1]), __float_as_uint(f0[0]), 0x0c0c0400u);
      *reinterpret_cast<uint16_t*>(base + kGroup) =
          (uint16_t)__builtin_amdgcn_perm(__float_as_uint(f1[1]), __float_as_uint(f1[0]), 0x0c0c0400u);
      *reinterpret_cast<uint16_t*>(base + 2 * kGroup) =
          (uint16_t)__builtin_amdgcn_perm(__float_as_uint(f2[1]), __float_as_uint(f2[0]), 0x0c0c0400u);
    }
    __syncthreads();  // B4: w limbs ready

    // (E) PV for this wave's channel tiles.
    v4i aw[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (arow_valid) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sm.wl[hm][im][16 * (2 * G + s)]);
        aw[s] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {
        aw[s] = v4i{0, 0, 0, 0};
      }
    }
    v4i tacc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) tacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[s], ones, tacc, 0, 0, 0);
    const uint32_t neglt =
        0u - (uint32_t)LV * (((uint32_t)tacc[0] << 14) + ((uint32_t)tacc[1] << 7) + (uint32_t)tacc[2]);
    const float vscale = W * (1.0f / (WMAX * 32768.0f));
#pragma unroll
    for (int c = 0; c < CTW; ++c) {
      const int ct = w * CTW + c;
      const uint8_t* vp = cur + Gm::KREC + (16 * ct + n) * Gm::VROW + G * Gm::LBV;
      uint32_t vw[Gm::LBV / 4];
#pragma unroll
      for (int k = 0; k < Gm::LBV / 4; ++k) vw[k] = reinterpret_cast<const uint32_t*>(vp)[k];
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[s], unpack16<VB>(&vw[s * (VB / 2)]), acc, 0, 0, 0);
      const uint32_t x = ((uint32_t)acc[0] << 14) + ((uint32_t)acc[1] << 7) + (uint32_t)acc[2];
      const int yv = (int)((x << 1) + neglt);
      o_acc[c] = fmaf((float)yv * vscale, h2f(cv16[16 * ct + n]), o_acc[c]);
    }
    if (more) store_stage(sm.buf[(it + 1) & 1]);
    __syncthreads();  // B0: next group staged; LDS areas free for reuse
  }

  // Partial of this split: m (replicated), l (sum over waves), o (disjoint
  // channel tiles per wave), straight to the workspace.
  const float lw = row16_sum(l_run);
  if (n == 0 && hvalid) sm.lsum[w][G] = lw;
  __syncthreads();
  if (hvalid) {
    const int hq_idx = kvh * GQ + G;
    const int64_t row = ((int64_t)b * a.hq + hq_idx) * a.nsplit + split;
#pragma unroll
    for (int c = 0; c < CTW; ++c) a.ws_o[row * D + 16 * (w * CTW + c) + n] = o_acc[c];
    if (w == 0 && n == 0) {
      float L = 0.f;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) L += sm.lsum[k][G];
      store_partial_ml(a, b, hq_idx, split, m_run, L);
    }
  }
}

// ---------------------------------------------------------------------------
// Exact split: the sink and the tail, fp16, original frame.  Exact split es
// covers exact tokens [128 es, 128 es + 128); wave w takes 32 of them in two
// rounds of 16; lane (token, quarter) holds a quarter of a K row and of a V
// row.  QK: fp32 FMAs against the LDS query; PV: V rows staged in LDS.
// ---------------------------------------------------------------------------
template <int D, int GQ>
__device__ void exact_split(ExactSmem<D, GQ>& sm, const DecodeArgs& a, int b, int kvh, int es, int split, int n) {
  constexpr int QD = D / 4;     // channels per lane (quarter row)
  constexpr int CPLX = D / 64;  // channels per lane in the PV part
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int quarter = l >> 4, tl = l & 15;
  for (int idx = tid; idx < GQ * D; idx += 256) {
    const int h = idx / D, j = idx % D;
    sm.qx[h][j] = __half2float(a.q[((int64_t)b * a.hq + kvh * GQ + h) * D + j]) * a.scale * kLog2e;
  }
  __syncthreads();
  const int n_sink = min(n, kSink);
  const int tau = n > kSink ? (n - kSink) % kGroup : 0;
  const int n_exact = max(0, n_sink + tau);
  const int64_t bh = (int64_t)b * a.c.hkv + kvh;

  float m_run[GQ], l_run[GQ], o[GQ][CPLX];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CPLX; ++c) o[h][c] = 0.f;
  }
  for (int round = 0; round < 2; ++round) {
    const int e0 = kGroup * es + 32 * w + kExactTok * round;
    const int e = e0 + tl;
    const bool valid = e < n_exact;
    float dot[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) dot[h] = 0.f;
    uint16_t* vrow = &sm.v[w][tl][quarter * QD];
    if (valid) {
      const size_t row = e < n_sink ? (size_t)(bh * kGroup + e) : (size_t)(bh * kGroup + (e - n_sink));
      const uint4* kp =
          reinterpret_cast<const uint4*>((e < n_sink ? a.c.sink_k : a.c.tail_k) + row * D + quarter * QD);
      const uint4* vp =
          reinterpret_cast<const uint4*>((e < n_sink ? a.c.sink_v : a.c.tail_v) + row * D + quarter * QD);
      uint4 kr[QD / 8], vr[QD / 8];
#pragma unroll
      for (int c = 0; c < QD / 8; ++c) {
        kr[c] = kp[c];
        vr[c] = vp[c];
      }
#pragma unroll
      for (int c = 0; c < QD / 8; ++c) reinterpret_cast<uint4*>(vrow)[c] = vr[c];
#pragma unroll
      for (int c = 0; c < QD / 8; ++c) {
        const uint32_t ws[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
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
    } else {
#pragma unroll
      for (int c = 0; c < QD / 8; ++c) reinterpret_cast<uint4*>(vrow)[c] = make_uint4(0, 0, 0, 0);
    }
    float pt[GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float lg = dot[h];
      lg += __shfl_xor(lg, 16, 64);
      lg += __shfl_xor(lg, 32, 64);
      lg = valid ? lg : -INFINITY;
      const float rmax = wave_max(lg);
      const float m_new = fmaxf(m_run[h], rmax);
      const float alpha = (m_run[h] == -INFINITY) ? 0.f : exp2f(m_run[h] - m_new);
      const float p = (valid && m_new != -INFINITY) ? exp2f(lg - m_new) : 0.f;
      pt[h] = p;
      l_run[h] = l_run[h] * alpha + wave_sum(quarter == 0 ? p : 0.f);
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
}

template <int D, int KB, int VB, int GQ>
union DecodeSmemU {
  RecSmem<D, KB, VB, GQ> rec;
  ExactSmem<D, GQ> ex;
};

template <int D, int KB, int VB, int GQ>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ DecodeSmemU<D, KB, VB, GQ> sm;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int n = a.c.seq_len[b];
  if (split < a.n_rec_splits)
    record_split<D, KB, VB, GQ>(sm.rec, a, b, kvh, split, n);
  else
    exact_split<D, GQ>(sm.ex, a, b, kvh, split - a.n_rec_splits, split, n);
}

// One workgroup (256 threads) per (query head, request): log-sum-exp merge of
// all splits, one inverse Hadamard of the record part, normalization.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int MAXS = 1024;  // splits handled per pass of the weight table
  __shared__ float wgt[MAXS];
  __shared__ float red[256];
  __shared__ float orot[D];
  __shared__ float oex[D];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t base = ((int64_t)b * a.hq + hq) * a.nsplit;
  float m = -INFINITY;
  for (int s = tid; s < a.nsplit; s += 256) m = fmaxf(m, a.ws_ml[2 * (base + s)]);
  red[tid] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float lsum = 0.f;
  for (int idx = tid; idx < D; idx += 256) {
    orot[idx] = 0.f;
    oex[idx] = 0.f;
  }
  constexpr int P = 256 / D;  // threads per channel
  const int j = tid % D, part = tid / D;
  float accr = 0.f, acce = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += MAXS) {
    const int cnt = min(MAXS, a.nsplit - s0);
    __syncthreads();
    for (int s = tid; s < cnt; s += 256) {
      const float ms = a.ws_ml[2 * (base + s0 + s)];
      const float f = (M == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - M);
      wgt[s] = f;
      lsum = fmaf(f, a.ws_ml[2 * (base + s0 + s) + 1], lsum);
    }
    __syncthreads();
    int s = part;
    for (; s + 7 * P < cnt; s += 8 * P) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = a.ws_o[(base + s0 + s + u * P) * D + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + s + u * P < a.n_rec_splits)
          accr = fmaf(wgt[s + u * P], v[u], accr);
        else
          acce = fmaf(wgt[s + u * P], v[u], acce);
      }
    }
    for (; s < cnt; s += P) {
      const float v = a.ws_o[(base + s0 + s) * D + j];
      if (s0 + s < a.n_rec_splits)
        accr = fmaf(wgt[s], v, accr);
      else
        acce = fmaf(wgt[s], v, acce);
    }
  }
  red[tid] = lsum;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float L = red[0];
  atomicAdd(&orot[j], accr);
  atomicAdd(&oex[j], acce);
  __syncthreads();
  // Inverse rotation of the record part (H symmetric): orot <- orot H.
  for (int st = 1; st < D; st <<= 1) {
    float x = 0.f, y = 0.f;
    if (tid < D) {
      x = orot[tid];
      y = orot[tid ^ st];
    }
    __syncthreads();
    if (tid < D) orot[tid] = (tid & st) ? y - x : x + y;
    __syncthreads();
  }
  if (tid < D) {
    const float rs = (D == 128) ? 0.08838834764831845f : 0.0625f;
    const float o = L > 0.f ? (orot[tid] * rs + oex[tid]) / L : 0.f;
    a.out[((int64_t)b * a.hq + hq) * D + tid] = o;
  }
}

DecodePlan plan_decode(int D, int hq, int hkv, int batch, int max_groups) {
  DecodePlan p;
  // About four workgroups per CU on 256 CUs, each walking a contiguous range
  // of groups of one (request, KV head).
  const int64_t pairs = (int64_t)batch * hkv;
  const int64_t target = 1024;
  p.n_exact_splits = 2;  // exact tokens [0,128) and [128,256)
  int gps = 1;
  if (max_groups > 0) {
    while (gps < max_groups) {
      const int64_t splits = (max_groups + gps - 1) / gps;
      if (pairs * (splits + p.n_exact_splits) <= target) break;
      ++gps;
    }
  }
  p.groups_per_split = gps;
  p.groups_per_wave = gps;
  p.n_rec_splits = max_groups > 0 ? (max_groups + gps - 1) / gps : 0;
  p.nsplit = p.n_rec_splits + p.n_exact_splits;
  const size_t rows = (size_t)batch * hq * p.nsplit;
  const size_t o_bytes = (rows * D * sizeof(float) + 255) & ~(size_t)255;
  p.ws_bytes = o_bytes + ((rows * 2 * sizeof(float) + 255) & ~(size_t)255);
  return p;
}

template <int D, int KB, int VB, int GQ>
static void launch_t(const DecodeArgs& a, int phases, hipStream_t st) {
  if (phases & 1)
    hipLaunchKernelGGL((decode_split_kernel<D, KB, VB, GQ>), dim3(a.nsplit, a.c.hkv, a.c.batch), dim3(256), 0, st,
                       a);
  if (phases & 2) hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(a.hq, a.c.batch), dim3(256), 0, st, a);
}

template <int D, int KB, int VB>
static void launch_g(int gq, const DecodeArgs& a, int phases, hipStream_t st) {
  if (gq == 1) launch_t<D, KB, VB, 1>(a, phases, st);
  else if (gq == 2) launch_t<D, KB, VB, 2>(a, phases, st);
  else launch_t<D, KB, VB, 4>(a, phases, st);
}

hipError_t launch_decode(int D, int kb, int vb, int gq, const DecodeArgs& a, int phases, hipStream_t st) {
  if (D == 128) {
    if (kb == 2 && vb == 2) launch_g<128, 2, 2>(gq, a, phases, st);
    else if (kb == 2 && vb == 4) launch_g<128, 2, 4>(gq, a, phases, st);
    else if (kb == 4 && vb == 2) launch_g<128, 4, 2>(gq, a, phases, st);
    else launch_g<128, 4, 4>(gq, a, phases, st);
  } else {
    if (kb == 2 && vb == 2) launch_g<256, 2, 2>(gq, a, phases, st);
    else if (kb == 2 && vb == 4) launch_g<256, 2, 4>(gq, a, phases, st);
    else if (kb == 4 && vb == 2) launch_g<256, 4, 2>(gq, a, phases, st);
    else launch_g<256, 4, 4>(gq, a, phases, st);
  }
  return hipGetLastError();
}

}  // namespace kvarn
