// KVarN decode attention on gfx950: the launch plan, the combine kernel and
// the dispatch to the split-kernel instances (decode_k<b>.hip, one per K
// code width).  The kernels themselves are in decode_impl.hpp.
#include "decode_impl.hpp"

namespace kvarn {

DecodePlan plan_decode(int D, int kb, int hq, int hkv, int batch, int max_groups, int resident_wgs, int cus) {
  DecodePlan p;
  // Each record workgroup is four independent waves; at run time each wave
  // takes an even share of its pair's sealed groups, at most groups_per_wave
  // of them (the grid is planned for the capacity max_groups).  The record
  // workgroups should be resident at once, so the smallest groups_per_wave
  // whose record grid fits the target maximises parallelism.
  //   * Few pairs: four one-round exact splits per pair, not counted in the
  //     target -- they are short and dispatched first, and the record
  //     workgroups that do not fit start as they retire.
  //   * Many pairs (four exact workgroups per pair would hold more than half
  //     of the resident slots): two two-round exact splits per pair, counted,
  //     so that every workgroup is resident at once; otherwise most record
  //     workgroups would start only after the exact ones retire.
  const int64_t pairs = (int64_t)batch * hkv;
  // Unless the exact workgroups need the third slot (many pairs), plan for at
  // most two record workgroups per CU: fewer, longer-running waves overlap
  // their groups' loads with the previous group's work and share the SIMDs
  // with fewer other waves.  Same-box A/B of the split kernel: Llama-3.1-8B
  // 11.45 -> 10.84 us (256 record workgroups of two groups per wave instead
  // of 512 of one), Phi-4 69.3 -> 65.5 us; at Qwen3-4B (many pairs) the cap
  // would cost 44.3 -> 45.8 us, so it is not applied there.  3-bit K codes
  // (bit-field extraction, a longer chain per group) keep three: the Llama
  // shape's 3-bit K preset 13.4 -> 12.5 us with 512 record workgroups of one
  // group per wave, where 2-bit K went 10.59 -> 11.35 us.
  // "Many pairs" is decided against the capped count: at the Phi-4 shape (80
  // pairs, three workgroups per CU) that gives two counted exact splits per
  // pair and 240 record workgroups, 66.0 us; decided against the uncapped
  // count it gave four uncounted exact splits and 480 record workgroups,
  // more workgroups than fit at once, 79 us.
  const int cap = kb == 3 ? 3 : 2;
  if (cus > 0 && !(2 * 4 * pairs > (int64_t)resident_wgs)) resident_wgs = std::min(resident_wgs, cap * cus);
  const bool many = 2 * 4 * pairs > (int64_t)resident_wgs;
  p.n_exact_splits = many ? 2 : 4;
  const int64_t target = many ? std::max<int64_t>(pairs, resident_wgs - 2 * pairs) : resident_wgs;
  int gpw = 1;
  if (max_groups > 0) {
    while (4 * gpw < max_groups) {
      const int64_t splits = (max_groups + 4 * gpw - 1) / (4 * gpw);
      if (pairs * splits <= target) break;
      ++gpw;
    }
  }
  int nrec = max_groups > 0 ? (max_groups + 4 * gpw - 1) / (4 * gpw) : 0;
  // A record grid just above a whole number k of workgroups per CU leaves a
  // few CUs with one more busy workgroup than the rest, and they finish last
  // (Llama-3.1-8B shape, capacity 257 groups: 520 record workgroups, 13.4 us;
  // 512, 11.3 us).  If dropping one split per pair reaches k per CU, drop it:
  // the waves share the groups actually sealed, so in the usual case (fewer
  // groups than the capacity) no wave gets more.  Larger excesses are kept:
  // there the extra waves carry their share of the traffic.
  if (cus > 0 && nrec > 1) {
    const int64_t r = pairs * nrec, k = r / cus;
    if (k >= 1 && r % cus != 0 && pairs * (nrec - 1) <= k * cus) {
      --nrec;
      gpw = (max_groups + 4 * nrec - 1) / (4 * nrec);
    }
  }
  p.groups_per_wave = gpw;
  p.groups_per_split = 4 * gpw;
  p.n_rec_splits = nrec;
  p.nsplit = p.n_rec_splits + p.n_exact_splits;
  // Grid order: when the record workgroups are one per CU at most (few
  // pairs), they go first, so that they are dispatched one to a CU before the
  // short exact ones fill in (Llama-3.1-8B shape, same-box A/B: split kernel
  // 10.84 -> 10.53 us, 3-bit K 14.2 -> 13.5 us).  Otherwise the exact ones go
  // first: with two record workgroups per CU (D 256 long context) record-first
  // was 1.2% slower, and with many pairs (Qwen3-4B) it gained nothing.
  p.record_first = !many && cus > 0 && pairs * nrec <= cus;
  const size_t rows = (size_t)batch * hq * p.nsplit;
  const size_t o_bytes = (rows * D * sizeof(float) + 255) & ~(size_t)255;
  p.ws_bytes = o_bytes + ((rows * 2 * sizeof(float) + 255) & ~(size_t)255);
  return p;
}

int decode_cu_count() {
  static std::atomic<int> cache[16];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 16 && (cus = cache[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 16) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int decode_resident_wgs(int D, int kb, int vb, int gq) {
  // Cached per device and kernel instance: [device][D][kb][vb][gq].
  static std::atomic<int> cache[16][2][6][6][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kMaxResidentWgs;
  const int di = D == 128 ? 0 : 1, ki = width_index(kb), vi = width_index(vb), gi = gq == 1 ? 0 : gq == 2 ? 1 : 2;
  std::atomic<int>* slot = dev < 16 ? &cache[dev][di][ki][vi][gi] : nullptr;
  int r = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (r > 0) return r;
  r = kb == 2   ? resident_split_k2(D, vb, gq, dev)
      : kb == 3 ? resident_split_k3(D, vb, gq, dev)
      : kb == 4 ? resident_split_k4(D, vb, gq, dev)
      : kb == 5 ? resident_split_k5(D, vb, gq, dev)
      : kb == 6 ? resident_split_k6(D, vb, gq, dev)
                : resident_split_k8(D, vb, gq, dev);
  r = r > 0 ? std::min(r, kMaxResidentWgs) : kMaxResidentWgs;
  if (slot) slot->store(r, std::memory_order_relaxed);
  return r;
}

hipError_t launch_decode(int D, int kb, int vb, int gq, const DecodeArgs& a, int phases, hipStream_t st) {
  if (phases & 1) {
    hipError_t e = kb == 2   ? launch_split_k2(D, vb, gq, a, st)
                   : kb == 3 ? launch_split_k3(D, vb, gq, a, st)
                   : kb == 4 ? launch_split_k4(D, vb, gq, a, st)
                   : kb == 5 ? launch_split_k5(D, vb, gq, a, st)
                   : kb == 6 ? launch_split_k6(D, vb, gq, a, st)
                             : launch_split_k8(D, vb, gq, a, st);
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    // First batch sized to the splits (clamped loads past the last split
    // repeat it; fewer of them with few splits, e.g. 6 at B 16).
    const dim3 grid(a.hq, a.c.batch);
    const int ns = a.nsplit;
#define KVARN_COMBINE(d)                                                                                  \
  do {                                                                                                    \
    if (ns <= 8) hipLaunchKernelGGL((decode_combine_kernel<d, 2>), grid, dim3(256), 0, st, a);           \
    else if (ns <= 20) hipLaunchKernelGGL((decode_combine_kernel<d, 5>), grid, dim3(256), 0, st, a);     \
    else if (ns <= 40) hipLaunchKernelGGL((decode_combine_kernel<d, 10>), grid, dim3(256), 0, st, a);    \
    else hipLaunchKernelGGL((decode_combine_kernel<d, 20>), grid, dim3(256), 0, st, a);                  \
  } while (0)
    if (D == 128) KVARN_COMBINE(128);
    else KVARN_COMBINE(256);
#undef KVARN_COMBINE
  }
  return hipGetLastError();
}

}  // namespace kvarn
