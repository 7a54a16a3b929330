// Decode split-kernel instances for 2-bit K records: every V width, head
// dimension (128, 256), query heads per KV head (1, 2, 4), contiguous and
// paged records.
#include "decode_impl.hpp"

namespace kvarn {

hipError_t launch_split_k2(int D, int vb, int gq, const DecodeArgs& a, hipStream_t st) {
  return launch_split_kb<2>(D, vb, gq, a, st);
}

int resident_split_k2(int D, int vb, int gq, int dev) { return resident_split_kb<2>(D, vb, gq, dev); }

#ifdef KVARN_WAVE_TRACE
hipError_t trace_io_decode_k2(void* host, size_t bytes) { return trace_io_local(host, bytes); }
#endif

}  // namespace kvarn
