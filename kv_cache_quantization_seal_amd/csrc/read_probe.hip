// Streaming-read probe: a measurement aid with no KVarN computation, built as
// its own library (libkvarn_probe.so) beside the KVarN library.  Timing it
// gives the achievable streaming-read bandwidth of the device, reported next
// to the HBM peak for the decode kernel.
//
// Each thread reads 16-byte pieces in a grid-stride loop, four independent
// nontemporal loads per trip, and folds them into one word that is stored
// only if it equals an improbable constant (the loads stay live; the kernel
// writes nothing in practice).  Launched with 32 workgroups per CU: measured
// over 4 GiB, nontemporal loads and the larger grid took the probe from 5.5
// to 6.6 TB/s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace {

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16, uint32_t* sink) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4* q = reinterpret_cast<const u4*>(p);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u4 x0 = __builtin_nontemporal_load(q + i), x1 = __builtin_nontemporal_load(q + i + stride);
    const u4 x2 = __builtin_nontemporal_load(q + i + 2 * stride), x3 = __builtin_nontemporal_load(q + i + 3 * stride);
    a0 ^= x0.x ^ x0.y ^ x0.z ^ x0.w;
    a1 ^= x1.x ^ x1.y ^ x1.z ^ x1.w;
    a2 ^= x2.x ^ x2.y ^ x2.z ^ x2.w;
    a3 ^= x3.x ^ x3.y ^ x3.z ^ x3.w;
  }
  for (; i < n16; i += stride) {
    const u4 x = q[i];
    a0 ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  const uint32_t a = a0 ^ a1 ^ a2 ^ a3;
  if (a == 0x9E3779B9u) sink[0] = a;
}

}  // namespace

// Reads `bytes` bytes at `buf` (device, 16-byte aligned, bytes a multiple of
// 16); `sink` (device, 4-byte aligned) is written only for an improbable
// combination of a thread's data.  Returns 0, or -1 for bad arguments (checked
// before anything is queued), or -5 if the launch failed.
extern "C" int kvarn_probe_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return 0;
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15) ||
      (reinterpret_cast<uintptr_t>(sink) & 3))
    return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -5;
  const size_t n16 = bytes / 16;
  const size_t want = (n16 + 255) / 256;
  const unsigned grid = (unsigned)std::min<size_t>(want, (size_t)std::max(cus, 1) * 32);
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(buf), n16, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
