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
// Record part (one wavefront per 128-token group, GQ query heads sharing it):
//   logit_t = s^K_t * sum_j q~_j (code_tj - mid) with q~ = q_r * c^K * scale,
//   w_t = p_t * s^V_t,   o_rot_j += c^V_j * sum_t w_t (code_tj - mid).
// Both sums run on v_mfma_i32_16x16x64_i8.  The codes are exact int8
// operands.  q~ (per group, per head) and w (per group, per head) are split
// into three int8 limbs x ~ E (a0 + a1/254 + a2/254^2) with |x - ...| <=
// E/(2*254^2) relative to the group maximum E/127; the 16 MFMA rows carry
// (head, limb) pairs, so one lane ends up with all limbs of one head and
// recombines them exactly: 2 C_i - (2^b - 1) S_i is an exact integer (S_i =
// limb sum), converted once to fp32.
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
//   tok(nt, n) = 16 (n/2) + unpack_index<VB>(8 (n%2) + nt) makes the w limbs
//   of one lane land on 8 consecutive LDS bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace kvarn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;

template <int D, int GQ>
struct alignas(16) DecodeSmem {
  alignas(16) float qx[GQ][D];  // scaled query (original frame, then rotated in place)
  union alignas(16) {
    struct {
      alignas(16) uint8_t ql[kWaves][4][3][D];        // q~ limbs in operand order
      alignas(16) uint8_t wl[kWaves][4][3][kGroup];   // w limbs in operand order
      alignas(16) uint16_t meta[kWaves][2][kGroup + D];  // [K|V][s(128) c(D)] fp16
    } rec;
    struct {
      alignas(16) uint16_t v[kWaves][32][D + 8];  // V rows of the wave's 32 exact tokens (fp16)
      alignas(16) float p[kWaves][32][4];          // softmax numerators [token][head]
    } ex;
  } u;
  float mm[kWaves][GQ];
  float ll[kWaves][GQ];
  float oo[kWaves][GQ][D];
};

template <int VB>
__device__ __forceinline__ int tok_of(int nt, int n) {
  return 16 * (n >> 1) + unpack_index<VB>(8 * (n & 1) + nt);
}

template <int NBYTES>
__device__ __forceinline__ void load_bytes(uint32_t* dst, const uint8_t* src) {
  if constexpr (NBYTES == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(src);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
#pragma unroll
    for (int k = 0; k < NBYTES / 16; ++k) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[k];
      dst[4 * k] = v.x;
      dst[4 * k + 1] = v.y;
      dst[4 * k + 2] = v.z;
      dst[4 * k + 3] = v.w;
    }
  }
}

// Merge the per-wave (m, l, o) of the workgroup and write one partial.
template <int D, int GQ>
__device__ __forceinline__ void merge_and_store(DecodeSmem<D, GQ>& sm, const DecodeArgs& a, int b, int kvh,
                                                int split) {
  __syncthreads();
  for (int idx = threadIdx.x; idx < GQ * D; idx += blockDim.x) {
    const int h = idx / D, ch = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.mm[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.mm[w][h];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
        L = fmaf(f, sm.ll[w][h], L);
        O = fmaf(f, sm.oo[w][h][ch], O);
      }
    }
    const int64_t row = ((int64_t)b * a.hq + kvh * GQ + h) * a.nsplit + split;
    a.ws_o[row * D + ch] = O;
    if (ch == 0) {
      a.ws_ml[2 * row] = M;
      a.ws_ml[2 * row + 1] = L;
    }
  }
}

template <int D, int KB, int VB, int GQ>
__device__ void record_split(DecodeSmem<D, GQ>& sm, const DecodeArgs& a, int b, int kvh, int split, int nseq) {
  constexpr int KS = D / 64;              // QK K-steps
  constexpr int CPL = D / 16;             // q~ values produced per lane
  constexpr int LBK = KS * 2 * KB;        // K-code bytes per lane per token
  constexpr int LBV = 2 * 2 * VB;         // V-code bytes per lane per channel
  constexpr int KROW = D * KB / 8;        // bytes per token row of K codes
  constexpr int VROW = kGroup * VB / 8;   // bytes per channel row of V codes
  constexpr int KCODE = kGroup * D * KB / 8;
  constexpr int VCODE = kGroup * D * VB / 8;
  constexpr int NCT = D / 16;             // PV N-tiles
  constexpr int LK = (1 << KB) - 1;
  constexpr int LV = (1 << VB) - 1;
  constexpr int META_CHUNKS = (kGroup + D) * 2 / 16;  // 16-byte chunks per K or V meta

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int G = l >> 4, n = l & 15;
  const bool hvalid = G < GQ;

  // Rotate the scaled query in place: qx <- qx H_D / sqrt(D).
  for (int s = 1; s < D; s <<= 1) {
    for (int idx = threadIdx.x; idx < GQ * D / 2; idx += blockDim.x) {
      const int h = idx / (D / 2), r = idx % (D / 2);
      const int lo = ((r & ~(s - 1)) << 1) | (r & (s - 1));
      const float x0 = sm.qx[h][lo], x1 = sm.qx[h][lo + s];
      sm.qx[h][lo] = x0 + x1;
      sm.qx[h][lo + s] = x0 - x1;
    }
    __syncthreads();
  }
  const float rs = (D == 128) ? 0.08838834764831845f : 0.0625f;
  float qr[CPL];
  int chq[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const int ob = n * CPL + e;
    chq[e] = 16 * (ob >> 4) + unpack_index<KB>(ob & 15);
    qr[e] = hvalid ? sm.qx[G][chq[e]] * rs : 0.f;
  }

  const int n_groups = nseq > kSink ? min((nseq - kSink) / kGroup, a.c.max_groups) : 0;
  const int g0 = split * a.groups_per_split;
  const int g1 = min(g0 + a.groups_per_split, n_groups);

  float m_run = -INFINITY, l_run = 0.f;
  float o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = 0.f;

  const int mrow = n;  // A-operand row of this lane: (head mrow/4, limb mrow%4)
  const int hm = mrow >> 2, im = mrow & 3;
  const bool arow_valid = hm < GQ && im < 3;
  uint8_t* qlw = &sm.u.rec.ql[w][0][0][0];
  uint8_t* wlw = &sm.u.rec.wl[w][0][0][0];
  uint16_t* metaw = &sm.u.rec.meta[w][0][0];

  for (int g = g0 + w; g < g1; g += kWaves) {
    const uint8_t* rec = a.c.records + (((int64_t)b * a.c.hkv + kvh) * a.c.max_groups + g) * a.c.group_bytes;
    const uint8_t* vrec = rec + a.c.rec_k_bytes;
    // Scale metadata -> LDS (K: s, c; V: s, c), 16-byte chunks.
    for (int i = l; i < 2 * META_CHUNKS; i += kWave) {
      const int kind = i / META_CHUNKS, c = i % META_CHUNKS;
      const uint8_t* srcm = kind ? vrec + VCODE : rec + KCODE;
      reinterpret_cast<uint4*>(metaw + kind * (kGroup + D))[c] = reinterpret_cast<const uint4*>(srcm)[c];
    }
    // Code operands straight to registers.
    uint32_t kc[8][LBK / 4];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      load_bytes<LBK>(kc[nt], rec + tok_of<VB>(nt, n) * KROW + G * LBK);
    uint32_t vc[NCT][LBV / 4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) load_bytes<LBV>(vc[ct], vrec + (16 * ct + n) * VROW + G * LBV);
    wave_sync();

    // q~ = q_r * c^K for this lane's channels, limbs into LDS.
    const uint16_t* ck = metaw + kGroup;
    float y[CPL];
    float ymax = 0.f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      y[e] = qr[e] * h2f(ck[chq[e]]);
      ymax = fmaxf(ymax, fabsf(y[e]));
    }
    const float E = row16_max(ymax);
    const float qinv = E > 0.f ? 127.0f / E : 0.f;
    float ssum0 = 0.f, ssum1 = 0.f, ssum2 = 0.f;
    if (hvalid) {
#pragma unroll
      for (int e4 = 0; e4 < CPL / 4; ++e4) {
        float l0[4], l1[4], l2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          limbs3(y[4 * e4 + e] * qinv, l0[e], l1[e], l2[e]);
          ssum0 += l0[e];
          ssum1 += l1[e];
          ssum2 += l2[e];
        }
        uint32_t* q0 = reinterpret_cast<uint32_t*>(qlw + (G * 3 + 0) * D + n * CPL) + e4;
        uint32_t* q1 = reinterpret_cast<uint32_t*>(qlw + (G * 3 + 1) * D + n * CPL) + e4;
        uint32_t* q2 = reinterpret_cast<uint32_t*>(qlw + (G * 3 + 2) * D + n * CPL) + e4;
        *q0 = pack4_i8(l0[0], l0[1], l0[2], l0[3]);
        *q1 = pack4_i8(l1[0], l1[1], l1[2], l1[3]);
        *q2 = pack4_i8(l2[0], l2[1], l2[2], l2[3]);
      }
    }
    const int S0 = (int)row16_sum(ssum0), S1 = (int)row16_sum(ssum1), S2 = (int)row16_sum(ssum2);
    wave_sync();
    v4i aq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (arow_valid) {
        const uint4 v = *reinterpret_cast<const uint4*>(qlw + (hm * 3 + im) * D + 16 * (G * KS + s));
        aq[s] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {
        aq[s] = v4i{0, 0, 0, 0};
      }
    }

    // QK on MFMA; recombine the limbs into base-2 logits.
    const uint16_t* sk = metaw;
    const uint16_t* sv = metaw + (kGroup + D);
    const float kscale = E * (0.5f / 127.0f);
    float logit[8];
    float gmax = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq[s], unpack16<KB>(&kc[nt][s * (2 * KB / 4)]), acc, 0, 0, 0);
      const float f0 = (float)(2 * acc[0] - LK * S0);
      const float f1 = (float)(2 * acc[1] - LK * S1);
      const float f2 = (float)(2 * acc[2] - LK * S2);
      const float f = fmaf(fmaf(f2, 1.0f / 254.0f, f1), 1.0f / 254.0f, f0);
      const int tok = tok_of<VB>(nt, n);
      logit[nt] = hvalid ? f * kscale * h2f(sk[tok]) : -INFINITY;
      gmax = fmaxf(gmax, logit[nt]);
    }
    gmax = row16_max(gmax);
    const float m_new = fmaxf(m_run, gmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f, wmax = 0.f;
    float wv[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float p = hvalid ? exp2f(logit[nt] - m_new) : 0.f;
      psum += p;
      wv[nt] = p * h2f(sv[tok_of<VB>(nt, n)]);
      wmax = fmaxf(wmax, wv[nt]);
    }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o_acc[ct] *= alpha;
    const float W = row16_max(wmax);
    const float winv = W > 0.f ? 127.0f / W : 0.f;
    float t0 = 0.f, t1 = 0.f, t2 = 0.f;
    {
      float l0[8], l1[8], l2[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        limbs3(wv[nt] * winv, l0[nt], l1[nt], l2[nt]);
        t0 += l0[nt];
        t1 += l1[nt];
        t2 += l2[nt];
      }
      if (hvalid) {
        uint2* w0 = reinterpret_cast<uint2*>(wlw + (G * 3 + 0) * kGroup + 8 * n);
        uint2* w1 = reinterpret_cast<uint2*>(wlw + (G * 3 + 1) * kGroup + 8 * n);
        uint2* w2 = reinterpret_cast<uint2*>(wlw + (G * 3 + 2) * kGroup + 8 * n);
        *w0 = make_uint2(pack4_i8(l0[0], l0[1], l0[2], l0[3]), pack4_i8(l0[4], l0[5], l0[6], l0[7]));
        *w1 = make_uint2(pack4_i8(l1[0], l1[1], l1[2], l1[3]), pack4_i8(l1[4], l1[5], l1[6], l1[7]));
        *w2 = make_uint2(pack4_i8(l2[0], l2[1], l2[2], l2[3]), pack4_i8(l2[4], l2[5], l2[6], l2[7]));
      }
    }
    const int T0 = (int)row16_sum(t0), T1 = (int)row16_sum(t1), T2 = (int)row16_sum(t2);
    wave_sync();
    v4i aw[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (arow_valid) {
        const uint4 v = *reinterpret_cast<const uint4*>(wlw + (hm * 3 + im) * kGroup + 16 * (2 * G + s));
        aw[s] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {
        aw[s] = v4i{0, 0, 0, 0};
      }
    }
    // PV on MFMA: rows (head G, limb i), column channel 16 ct + n.
    const uint16_t* cv = sv + kGroup;
    const float vscale = W * (0.5f / 127.0f);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw[s], unpack16<VB>(&vc[ct][s * (2 * VB / 4)]), acc, 0, 0, 0);
      const float f0 = (float)(2 * acc[0] - LV * T0);
      const float f1 = (float)(2 * acc[1] - LV * T1);
      const float f2 = (float)(2 * acc[2] - LV * T2);
      const float f = fmaf(fmaf(f2, 1.0f / 254.0f, f1), 1.0f / 254.0f, f0);
      o_acc[ct] = fmaf(f * vscale, h2f(cv[16 * ct + n]), o_acc[ct]);
    }
    wave_sync();  // LDS areas are rewritten by the next group
  }

  const float l_tot = row16_sum(l_run);
  if (hvalid) {
    if (n == 0) {
      sm.mm[w][G] = m_run;
      sm.ll[w][G] = l_tot;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) sm.oo[w][G][16 * ct + n] = o_acc[ct];
  }
}

// Exact part: the sink and the tail, fp16, original frame.  Exact split es
// covers exact tokens [128 es, 128 es + 128); wave w takes 32 of them, lane
// (token, half) holds half a K row and half a V row.  QK: fp32 FMAs against
// the LDS query; PV: V rows staged in LDS, lane = channel group.
template <int D, int GQ>
__device__ void exact_split(DecodeSmem<D, GQ>& sm, const DecodeArgs& a, int b, int kvh, int es, int n) {
  constexpr int HALF = D / 2;
  constexpr int CPLX = D / 64;  // channels per lane in the PV part
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int half = l >> 5, tl = l & 31;
  const int n_sink = min(n, kSink);
  const int tau = n > kSink ? (n - kSink) % kGroup : 0;
  const int n_exact = max(0, n_sink + tau);
  const int64_t bh = (int64_t)b * a.c.hkv + kvh;
  const int e = kGroup * es + 32 * w + tl;
  const bool valid = e < n_exact;
  float dot[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) dot[h] = 0.f;
  uint16_t* vrow = &sm.u.ex.v[w][tl][half * HALF];
  if (valid) {
    const size_t row = e < n_sink ? (size_t)(bh * kGroup + e) : (size_t)(bh * kGroup + (e - n_sink));
    const uint4* kp = reinterpret_cast<const uint4*>((e < n_sink ? a.c.sink_k : a.c.tail_k) + row * D + half * HALF);
    const uint4* vp = reinterpret_cast<const uint4*>((e < n_sink ? a.c.sink_v : a.c.tail_v) + row * D + half * HALF);
    uint4 kr[HALF / 8], vr[HALF / 8];
#pragma unroll
    for (int c = 0; c < HALF / 8; ++c) {
      kr[c] = kp[c];
      vr[c] = vp[c];
    }
#pragma unroll
    for (int c = 0; c < HALF / 8; ++c) reinterpret_cast<uint4*>(vrow)[c] = vr[c];
#pragma unroll
    for (int c = 0; c < HALF / 8; ++c) {
      const uint32_t ws[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
      for (int h = 0; h < GQ; ++h) {
        const float4 qa = *reinterpret_cast<const float4*>(&sm.qx[h][half * HALF + 8 * c]);
        const float4 qb = *reinterpret_cast<const float4*>(&sm.qx[h][half * HALF + 8 * c + 4]);
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
    for (int c = 0; c < HALF / 8; ++c) reinterpret_cast<uint4*>(vrow)[c] = make_uint4(0, 0, 0, 0);
  }
  float mh[GQ], lh[GQ];
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    const float lg = valid ? dot[h] + __shfl_xor(dot[h], 32, 64) : -INFINITY;
    mh[h] = wave_max(lg);
    const float p = (valid && mh[h] != -INFINITY) ? exp2f(lg - mh[h]) : 0.f;
    lh[h] = wave_sum(half == 0 ? p : 0.f);
    if (half == 0) sm.u.ex.p[w][tl][h] = p;
  }
  wave_sync();
  float o[GQ][CPLX];
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int c = 0; c < CPLX; ++c) o[h][c] = 0.f;
  const int nt = min(32, max(0, n_exact - (kGroup * es + 32 * w)));
  for (int t = 0; t < nt; ++t) {
    const float4 pv = *reinterpret_cast<const float4*>(&sm.u.ex.p[w][t][0]);
    const float ph[4] = {pv.x, pv.y, pv.z, pv.w};
    float vf[CPLX];
    if constexpr (CPLX == 2) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(&sm.u.ex.v[w][t][2 * l]);
      vf[0] = h2f((uint16_t)(x & 0xFFFFu));
      vf[1] = h2f((uint16_t)(x >> 16));
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(&sm.u.ex.v[w][t][4 * l]);
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
#pragma unroll
  for (int h = 0; h < GQ; ++h) {
    if (l == 0) {
      sm.mm[w][h] = mh[h];
      sm.ll[w][h] = lh[h];
    }
#pragma unroll
    for (int c = 0; c < CPLX; ++c) sm.oo[w][h][CPLX * l + c] = o[h][c];
  }
}

template <int D, int KB, int VB, int GQ>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ DecodeSmem<D, GQ> sm;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int n = a.c.seq_len[b];
  // Scaled query (log2 domain) of the GQ heads that share KV head kvh.
  for (int idx = threadIdx.x; idx < GQ * D; idx += blockDim.x) {
    const int h = idx / D, j = idx % D;
    const float qv = __half2float(a.q[((int64_t)b * a.hq + kvh * GQ + h) * D + j]);
    sm.qx[h][j] = qv * a.scale * kLog2e;
  }
  for (int idx = threadIdx.x; idx < kWaves * GQ; idx += blockDim.x) {
    sm.mm[idx / GQ][idx % GQ] = -INFINITY;
    sm.ll[idx / GQ][idx % GQ] = 0.f;
  }
  for (int idx = threadIdx.x; idx < kWaves * GQ * D; idx += blockDim.x) (&sm.oo[0][0][0])[idx] = 0.f;
  __syncthreads();
  if (split < a.n_rec_splits)
    record_split<D, KB, VB, GQ>(sm, a, b, kvh, split, n);
  else
    exact_split<D, GQ>(sm, a, b, kvh, split - a.n_rec_splits, n);
  merge_and_store<D, GQ>(sm, a, b, kvh, split);
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
  // Global max over splits.
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
  // Channel partial sums: thread (j, part) sums splits part, part + P, ...
  constexpr int P = 256 / D;  // 2 for D = 128, 1 for D = 256
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
        const int ss = s0 + s + u * P;
        if (ss < a.n_rec_splits)
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
  const int64_t total = (int64_t)batch * hkv * max_groups;
  const int64_t target_waves = 2048;  // 256 CUs x 8 waves
  int gpw = (int)((total + target_waves - 1) / target_waves);
  if (gpw < 1) gpw = 1;
  p.groups_per_wave = gpw;
  p.groups_per_split = kWaves * gpw;
  p.n_rec_splits = max_groups > 0 ? (max_groups + p.groups_per_split - 1) / p.groups_per_split : 0;
  p.n_exact_splits = 2;  // exact tokens [0,128) and [128,256)
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
