// Per-wave phase timestamps, compiled in only with KVARN_WAVE_TRACE (the
// trace build, libkvarn_trace.so); in the product library every call below
// is an empty inline function.
//
// Record of wave slot s (kTraceWords 64-bit words):
//   [0]              hardware ids: HW_ID register (low 32 bits) and XCC_ID
//                    (high 32 bits) of the wave
//   [1]              core-clock counter at the start of the wave
//   [2 .. 2+kPhases) real-time counter (100 MHz) at phase marks 0..kPhases-1
//   [kTraceWords-1]  core-clock counter at the last mark
// A mark that a wave does not reach stays 0 (the host clears the buffer
// before a traced launch).  Only lane 0 of a wave writes, with ordinary
// vector stores.  Slots past kTraceSlots are dropped.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

constexpr int kTracePhases = 12;
constexpr int kTraceWords = 16;
constexpr int kTraceSlots = 32768;

#ifdef KVARN_WAVE_TRACE
// One buffer per translation unit (each kernel source has its own).
static __device__ uint64_t g_trace[kTraceSlots * kTraceWords];

// Host: copy the buffer of this translation unit to `host` (bytes <= its
// size), or clear it (host NULL).  Synchronous.
static inline hipError_t trace_io_local(void* host, size_t bytes) {
  const size_t full = sizeof(uint64_t) * kTraceSlots * kTraceWords;
  if (bytes > full) bytes = full;
  if (!host) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_trace));
    if (e != hipSuccess) return e;
    e = hipMemset(p, 0, full);
    if (e != hipSuccess) return e;
    return hipDeviceSynchronize();
  }
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_trace), bytes, 0, hipMemcpyDeviceToHost);
}

__device__ __forceinline__ void trace_begin(int slot) {
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t ct = __builtin_amdgcn_s_memtime();
  const uint64_t rt = __builtin_amdgcn_s_memrealtime();
  const uint32_t hw = __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));   // HW_ID
  const uint32_t xcc = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11));  // XCC_ID
  if ((threadIdx.x & 63) == 0 && slot >= 0 && slot < kTraceSlots) {
    uint64_t* r = g_trace + (size_t)slot * kTraceWords;
    r[0] = ((uint64_t)xcc << 32) | hw;
    r[1] = ct;
    r[2] = rt;
  }
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void trace_mark(int slot, int phase) {
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t rt = __builtin_amdgcn_s_memrealtime();
  const uint64_t ct = __builtin_amdgcn_s_memtime();
  if ((threadIdx.x & 63) == 0 && slot >= 0 && slot < kTraceSlots && phase > 0 && phase < kTracePhases) {
    uint64_t* r = g_trace + (size_t)slot * kTraceWords;
    r[2 + phase] = rt;
    r[kTraceWords - 1] = ct;
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Loop kernels: core-clock cycles per phase, summed over the iterations of a
// wave, in place of the phase timestamps: record [2 + p] = cycles spent in
// phase p (p < kTracePhases), [1] / [kTraceWords-1] = the core-clock counter
// at the first / last mark.  phase_end(c, p) closes phase p at this point.
struct PhaseClock {
  uint64_t first, last;
  uint32_t acc[kTracePhases];
};
__device__ __forceinline__ void phase_start(PhaseClock& c) {
  __builtin_amdgcn_sched_barrier(0);
  c.first = c.last = __builtin_amdgcn_s_memtime();
#pragma unroll
  for (int p = 0; p < kTracePhases; ++p) c.acc[p] = 0;
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void phase_end(PhaseClock& c, int p) {
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t now = __builtin_amdgcn_s_memtime();
  c.acc[p] += (uint32_t)(now - c.last);
  c.last = now;
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void phase_store(int slot, const PhaseClock& c) {
  const uint32_t hw = __builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11));   // HW_ID
  const uint32_t xcc = __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (31 << 11));  // XCC_ID
  if ((threadIdx.x & 63) == 0 && slot >= 0 && slot < kTraceSlots) {
    uint64_t* r = g_trace + (size_t)slot * kTraceWords;
    r[0] = ((uint64_t)xcc << 32) | hw;
    r[1] = c.first;
#pragma unroll
    for (int p = 0; p < kTracePhases; ++p) r[2 + p] = c.acc[p];
    r[kTraceWords - 1] = c.last;
  }
}
#else
__device__ __forceinline__ void trace_begin(int) {}
__device__ __forceinline__ void trace_mark(int, int) {}
struct PhaseClock {};
__device__ __forceinline__ void phase_start(PhaseClock&) {}
__device__ __forceinline__ void phase_end(PhaseClock&, int) {}
__device__ __forceinline__ void phase_store(int, const PhaseClock&) {}
#endif

}  // namespace kvarn
